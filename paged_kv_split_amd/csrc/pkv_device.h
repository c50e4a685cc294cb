// pkv_device.h -- device helpers shared by the split kernels and the combine
// kernel of libpkv.so (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_internal.h"

namespace pkv {
namespace dev {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaxSplits = 256;  // = PKV_MAX_SPLITS

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 -> bf16 bits, round to nearest even (quiet NaN kept quiet)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 128-bit streaming load (K/V are read once per unit: non-temporal hint)
__device__ __forceinline__ uint4 load_stream(const uint4 *p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---- cross-lane primitives (DPP / permlane; semantics checked on gfx950) ----
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kMirror = 0x140;     // lane i <-> 15-i within 16
constexpr int kRor4 = 0x124;       // lane i receives lane (i-4) mod 16
constexpr int kRor8 = 0x128;       // lane i receives lane (i-8) mod 16 (= i xor 8)

struct OpSum {
  __device__ static float f(float a, float b) { return a + b; }
};
struct OpMax {
  __device__ static float f(float a, float b) { return fmaxf(a, b); }
};

template <class Op>
__device__ __forceinline__ float xor16(float x) {  // combine lanes i and i^16
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return Op::f(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
template <class Op>
__device__ __forceinline__ float xor32(float x) {  // combine lanes i and i^32
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return Op::f(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// Reduce over lane bits [LO, 6) of independent values.  Over the whole wave
// (LO = 0) every step pairs lane i with one partner that in turn pairs with
// lane i (xor 1, xor 2, mirror within 8, mirror within 16, xor 16, xor 32),
// and the operation is commutative, so every lane ends with the same
// bit-identical result.  With LO > 0 bits 2 and 3 are reduced by rotations,
// whose association differs from lane to lane.
template <int LO, class Op>
__device__ __forceinline__ float reduce_hi(float x) {
  if constexpr (LO <= 0) {
    x = Op::f(x, dpp<kXor1>(x));
    x = Op::f(x, dpp<kXor2>(x));
    x = Op::f(x, dpp<kHalfMirror>(x));  // quad sums: lanes 0-3 <-> 4-7
    x = Op::f(x, dpp<kMirror>(x));      // 8-lane sums: lanes 0-7 <-> 8-15
    x = xor16<Op>(x);
    return xor32<Op>(x);
  }
  if constexpr (LO <= 1) x = Op::f(x, dpp<kXor2>(x));
  if constexpr (LO <= 2) {  // bits 2 and 3 together: lanes i, i-4, i+4, i+8 (mod 16)
    x = Op::f(x, dpp<kRor4>(x));
    x = Op::f(x, dpp<kRor8>(x));
  } else if constexpr (LO <= 3) {
    x = Op::f(x, dpp<kRor8>(x));
  }
  if constexpr (LO <= 4) x = xor16<Op>(x);
  x = xor32<Op>(x);
  return x;
}

// ---- partial results: stores and loads at device scope ---------------------
// The split workgroups of one unit run on different XCDs, whose L2 caches are
// not kept coherent with each other.  Partials are therefore stored with
// device-scope stores (written through to the device-coherent level) and the
// merging workgroup reads them with device-scope loads (which do not hit
// possibly stale lines of its own L2), so no whole-cache writeback or
// invalidate is needed; completion of the stores (s_waitcnt) before the
// arrival counter's atomic orders them before the merge.
__device__ __forceinline__ void store_dev(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev2(float *p, float x, float y) {  // p 8-byte aligned
  const uint64_t u = (uint64_t)__float_as_uint(x) | ((uint64_t)__float_as_uint(y) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t *>(p), u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Four floats of a partial that another workgroup of the running launch
// reads (the in-kernel merge), p 16-byte aligned inside a.o_part.  With
// a.wide_part (a workspace under 2^31 bytes, so byte offsets fit 32 bits) one
// 16-byte raw buffer store with the sc1 cache policy -- written through to the
// device-coherent level, as the agent-scope atomic stores of store_dev2 are --
// over a resource that spans the workspace; otherwise two 8-byte agent-scope
// atomic stores.  Measured on MI355X (B = 256 ragged batch): each 8-byte
// write-through store cost a 32-byte memory write, 106 MB of writes per call
// for 39 MB of partials and outputs.
constexpr int kCpolSc1 = 16;               // cache-policy operand of the buffer builtins: sc1
constexpr int kRawBufferDword3 = 0x00020000;  // buffer resource word 3 for untyped (raw) access
__device__ __forceinline__ void store_part4(const DecodeArgs &a, float *p, float x, float y, float z, float w) {
  if (a.wide_part) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(a.o_part, 0, 0x7fffffff, kRawBufferDword3);
    typedef __attribute__((ext_vector_type(4))) int i32x4_t;
    const i32x4_t v = {__float_as_int(x), __float_as_int(y), __float_as_int(z), __float_as_int(w)};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)((p - a.o_part) * 4), 0, kCpolSc1);
  } else {
    store_dev2(p, x, y);
    store_dev2(p + 2, z, w);
  }
}

template <bool DEV>
__device__ __forceinline__ float2 load2(const float *p) {  // p 8-byte aligned
  if constexpr (DEV) {
    const uint64_t u =
        __hip_atomic_load(reinterpret_cast<uint64_t *>(const_cast<float *>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(__uint_as_float((uint32_t)u), __uint_as_float((uint32_t)(u >> 32)));
  } else {
    return *reinterpret_cast<const float2 *>(p);
  }
}

// The (sequence b, split s) pair of outer index p (0 <= p < B * S).  The
// split-major order puts every sequence's first split ahead of any second
// one, and rotating the sequences by 3s between splits gives each XCD (the
// pairs p, p + 8, ... land on one XCD) a mix of sequences and split
// positions, so ragged lengths and splits past a sequence's end spread over
// the XCDs rather than piling onto some.
__device__ __forceinline__ void decode_pair(int p, int n, int &b, int &s) {
  s = p / n;
  b = p - s * n + 3 * s;
  b %= n;
}

// Splits of a unit that hold keys: its rows see kmax keys at most.  At least
// one, so that a unit without keys still writes its (zero) output.
__device__ __forceinline__ int active_splits(const DecodeArgs &a, int kmax) {
  const int n = (kmax + a.chunk - 1) / a.chunk;
  return n < 1 ? 1 : (n > a.S ? a.S : n);
}

// Keys per page-table window: `cap` pages, a multiple of `step` keys, at
// least `step` and at most 2^30 (contiguous K/V has one page of up to 2^30
// keys per sequence).
__device__ __forceinline__ int window_keys(int cap, int page_shift, int step) {
  const int64_t w = ((int64_t)cap << page_shift) / step * step;
  if (w < step) return step;
  return w > ((int64_t)1 << 30) ? ((1 << 30) / step) * step : (int)w;
}

// The query rows of sequence b: its first token in q / out, its packed rows
// per kv head (G per query token) and its causal offset.  A varlen batch
// (a.cu_q) gives each sequence its own token count, at most a.q_len.
struct SeqRows {
  int64_t tok0;  // first token of the sequence in q and out
  int R;         // packed rows per kv head
  int cofs;      // causal offset (position of the sequence's first query token)
  bool causal;
};

// From the sequence's entries: kv length L, cu_q[b], cu_q[b + 1] (varlen)
// and causal_offsets[b] (when given).
template <bool CAUSAL>
__device__ __forceinline__ SeqRows seq_rows_of(const DecodeArgs &a, int b, int L, int c0, int c1, int co) {
  SeqRows r;
  if (a.cu_q) {
    int n = c1 - c0;
    n = n < 0 ? 0 : (n > a.q_len ? a.q_len : n);
    r.tok0 = c0;
    r.R = n * a.G;
  } else {
    r.tok0 = (int64_t)b * a.q_len;
    r.R = a.R;
  }
  r.cofs = -1;
  r.causal = false;
  if constexpr (CAUSAL) {
    if (a.causal_offsets) {
      r.cofs = co;
      r.causal = r.cofs >= 0;
    } else if (a.causal_offset == kCausalLast) {  // tokens at positions L - n .. L - 1
      r.cofs = L - r.R / a.G;
      r.causal = true;
    } else {
      r.cofs = a.causal_offset;
      r.causal = r.cofs >= 0;
    }
  }
  return r;
}

template <bool CAUSAL>
__device__ __forceinline__ SeqRows seq_rows(const DecodeArgs &a, int b, int L) {
  const int c0 = a.cu_q ? a.cu_q[b] : 0;
  const int c1 = a.cu_q ? a.cu_q[b + 1] : 0;
  const int co = (CAUSAL && a.causal_offsets) ? a.causal_offsets[b] : -1;
  return seq_rows_of<CAUSAL>(a, b, L, c0, c1, co);
}

// Keys packed row rr of the sequence may see: none past its rows; else its L
// keys, or with a causal offset those up to its token's position.
__device__ __forceinline__ int row_keys(const DecodeArgs &a, const SeqRows &sr, int L, int rr) {
  if (rr >= sr.R) return 0;
  int lr = L;
  if (sr.causal) {
    const int64_t cl = (int64_t)sr.cofs + rr / a.G + 1;
    if (cl < lr) lr = cl < 0 ? 0 : (int)cl;
  }
  return lr;
}

// ---- the schedule: which (sequence, split, kv-head group, row block) a
// split workgroup covers ---------------------------------------------------
struct Work {
  int b, s, hg, rg;  // sequence, split, kv-head group, row block
  int unit;          // (sequence, kv-head group, row block) unit: its arrival counter
  int L;             // the sequence's kv length
  SeqRows sr;
};

// Inclusive prefix sum over the 64 lanes of a wave, in DPP moves (no LDS
// permutes): shifts of 1, 2, 4 and 8 lanes within each row of 16 (lanes
// shifted in from before the row add 0) give every row's own prefix sums;
// then the last lane of row 0 (of row 2) is added to row 1 (row 3), and the
// last lane of row 1, by then the total of rows 0 and 1, to rows 2 and 3.
__device__ __forceinline__ int wave_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2 and 3
  return x;
}

constexpr int kExactPerLane = 4;  // sequences per lane of the exact schedule

// Exact schedule (up to 64 * kExactPerLane = 256 sequences): the work items are
// the (sequence, split, row block) triples that hold work -- row blocks with
// rows, and with the in-kernel merge or a single split only the splits up to
// the sequence's last key -- numbered sequence by sequence (split-major
// within a sequence, so the row blocks that read one K/V chunk are
// neighbours).  Every workgroup counts the items of all sequences (each lane
// a run of kExactPerLane at most, one round of loads, then a wave-wide prefix
// sum), so it knows their total N; XCD x (blocks x, x + 8, ...) takes items
// x * ceil(N / 8) onward, in order, and the blocks past them -- the grid is
// sized for a host-side bound -- exit at the end of the dispatch.
template <bool CAUSAL>
__device__ __forceinline__ bool work_exact(const DecodeArgs &a, int xcd, int slot, Work &w) {
  const int lane = threadIdx.x & 63;
  const int k = (a.B + 63) >> 6;
  const int b0 = lane * k;
  int Lq[kExactPerLane], c0q[kExactPerLane], c1q[kExactPerLane], coq[kExactPerLane];
#pragma unroll
  for (int j = 0; j < kExactPerLane; ++j) {
    const int b = b0 + j;
    const bool ok = j < k && b < a.B;
    Lq[j] = ok ? a.kv_lens[b] : 0;
    c0q[j] = ok && a.cu_q ? a.cu_q[b] : 0;
    c1q[j] = ok && a.cu_q ? a.cu_q[b + 1] : 0;
    coq[j] = ok && CAUSAL && a.causal_offsets ? a.causal_offsets[b] : -1;
  }
  const bool trimmed = a.fused || a.S == 1;  // splits past the last key get no item
  int items[kExactPerLane], rbs[kExactPerLane];
  int isum = 0, usum = 0;
#pragma unroll
  for (int j = 0; j < kExactPerLane; ++j) {
    items[j] = 0;
    rbs[j] = 0;
    if (j < k && b0 + j < a.B) {
      const SeqRows sr = seq_rows_of<CAUSAL>(a, b0 + j, Lq[j], c0q[j], c1q[j], coq[j]);
      rbs[j] = (sr.R + a.rp - 1) >> __builtin_ctz(a.rp);  // a.rp is a power of two
      const int ns = trimmed ? active_splits(a, row_keys(a, sr, Lq[j], sr.R - 1)) : a.S;
      items[j] = rbs[j] * ns;
    }
    isum += items[j];
    usum += rbs[j];
  }
  const int iscan = wave_scan(isum);
  const int uscan = wave_scan(usum);
  const int n_items = __builtin_amdgcn_readlane(iscan, 63);
  const int per = (n_items + 7) >> 3;
  const int kk = slot / a.inner;
  if (kk >= per) return false;
  const int v = xcd * per + kk;
  if (v >= n_items) return false;
  // the lane whose run holds item v, then the sequence within the run
  const uint64_t m = __builtin_amdgcn_ballot_w64(iscan > v);
  if (m == 0) return false;  // not reached: v < n_items
  const int sel = __builtin_ctzll(m);
  int ibase = __builtin_amdgcn_readlane(iscan - isum, sel);
  int ubase = __builtin_amdgcn_readlane(uscan - usum, sel);
  bool found = false;
  int jsel = 0, nitem = 0, nrb = 1;
#pragma unroll
  for (int j = 0; j < kExactPerLane; ++j) {
    const int c = __builtin_amdgcn_readlane(items[j], sel);
    const int r = __builtin_amdgcn_readlane(rbs[j], sel);
    if (!found) {
      if (v < ibase + c) {
        found = true;
        jsel = j;
        nitem = c;
        nrb = r;
      } else {
        ibase += c;
        ubase += r;
      }
    }
  }
  (void)nitem;
  int L = 0, c0 = 0, c1 = 0, co = -1;
#pragma unroll
  for (int j = 0; j < kExactPerLane; ++j) {
    if (j == jsel) {
      L = __builtin_amdgcn_readlane(Lq[j], sel);
      c0 = __builtin_amdgcn_readlane(c0q[j], sel);
      c1 = __builtin_amdgcn_readlane(c1q[j], sel);
      co = __builtin_amdgcn_readlane(coq[j], sel);
    }
  }
  const int jj = v - ibase;
  w.b = sel * k + jsel;
  w.s = jj / nrb;
  w.rg = jj - w.s * nrb;
  w.hg = slot - kk * a.inner;
  w.unit = (ubase + w.rg) * a.inner + w.hg;
  w.L = L;
  w.sr = seq_rows_of<CAUSAL>(a, w.b, L, c0, c1, co);
  return true;
}

// Longest first (a.lpt, with the exact schedule when every split past a
// sequence's last key is trimmed): the same items, dealt in decreasing key
// count so that the longest workgroups start first and the grid ends on short
// ones.  An item's keys are those of its split: whole chunks for every split
// but a sequence's last, which holds the rest.  Items fall in kLptBuckets
// buckets -- whole chunks, then kLptBuckets - 1 equal ranges of partial
// chunks -- taken from the largest down, sequence by sequence within a
// bucket (split-major, row blocks adjacent within a sequence).  Item v goes
// to block slot v / 8 of XCD v mod 8, so every XCD runs the same mix, longest
// first.  Per-bucket counts are summed over the wave exactly in fp32 (counts
// stay below 2^24); a wave prefix sum of the chosen bucket's counts then
// finds the lane and sequence of the item.
constexpr int kLptBuckets = 8;

template <bool CAUSAL>
__device__ __forceinline__ bool work_lpt(const DecodeArgs &a, int xcd, int slot, Work &w) {
  constexpr int NB = kLptBuckets;
  const int lane = threadIdx.x & 63;
  const int k = (a.B + 63) >> 6;
  const int b0 = lane * k;
  int Lq[kExactPerLane], c0q[kExactPerLane], c1q[kExactPerLane], coq[kExactPerLane];
#pragma unroll
  for (int j = 0; j < kExactPerLane; ++j) {
    const int b = b0 + j;
    const bool ok = j < k && b < a.B;
    Lq[j] = ok ? a.kv_lens[b] : 0;
    c0q[j] = ok && a.cu_q ? a.cu_q[b] : 0;
    c1q[j] = ok && a.cu_q ? a.cu_q[b + 1] : 0;
    coq[j] = ok && CAUSAL && a.causal_offsets ? a.causal_offsets[b] : -1;
  }
  // per sequence: row blocks, whole-chunk splits and the keys of its partial
  // split; their items counted first, so that a block past every item (the
  // grid is sized for a host-side bound) leaves before the buckets are formed
  const int lrp = __builtin_ctz(a.rp);  // a.rp is a power of two
  int rbs[kExactPerLane], nfull[kExactPerLane], remq[kExactPerLane];
  int isum = 0, usum = 0;
#pragma unroll
  for (int j = 0; j < kExactPerLane; ++j) {
    rbs[j] = 0;
    nfull[j] = 0;
    remq[j] = -1;   // -1: no partial split
    if (j < k && b0 + j < a.B) {
      const SeqRows sr = seq_rows_of<CAUSAL>(a, b0 + j, Lq[j], c0q[j], c1q[j], coq[j]);
      rbs[j] = (sr.R + a.rp - 1) >> lrp;
      const int kmax = sr.R > 0 ? row_keys(a, sr, Lq[j], sr.R - 1) : 0;
      if (kmax <= 0) {  // no key: one split that writes zero rows (bucket 0)
        remq[j] = 0;
      } else {
        nfull[j] = kmax / a.chunk;
        const int rem = kmax - nfull[j] * a.chunk;
        if (rem > 0) remq[j] = rem;
      }
    }
    isum += rbs[j] * (nfull[j] + (remq[j] >= 0 ? 1 : 0));
    usum += rbs[j];
  }
  const int n_items = (int)reduce_hi<0, OpSum>((float)isum);  // exact: counts stay below 2^24
  const int kk = slot / a.inner;
  const int v = kk * 8 + xcd;
  if (v >= n_items) return false;
  // bucket of each partial split: floor(rem * (NB - 1) / chunk) (rem < chunk;
  // in 32 bits while chunk * (NB - 1) fits, the branch being uniform)
  int pbk[kExactPerLane];
  int cnt[NB];
#pragma unroll
  for (int q = 0; q < NB; ++q) cnt[q] = 0;
#pragma unroll
  for (int j = 0; j < kExactPerLane; ++j) {
    pbk[j] = -1;
    if (remq[j] == 0) {
      pbk[j] = 0;
    } else if (remq[j] > 0) {
      pbk[j] = a.chunk < (INT32_MAX / (NB - 1)) ? remq[j] * (NB - 1) / a.chunk
                                                : (int)(((int64_t)remq[j] * (NB - 1)) / a.chunk);
    }
#pragma unroll
    for (int q = 0; q < NB; ++q) cnt[q] += (q == NB - 1 ? nfull[j] * rbs[j] : 0) + (q == pbk[j] ? rbs[j] : 0);
  }
  const int uscan = wave_scan(usum);
  int tot[NB];
#pragma unroll
  for (int q = 0; q < NB; ++q) tot[q] = (int)reduce_hi<0, OpSum>((float)cnt[q]);
  // the bucket of item v (whole chunks first, then the partial buckets from the largest)
  int jv = 0, ov = v;
  bool got = false;
#pragma unroll
  for (int q = NB - 1; q >= 0; --q) {
    if (!got) {
      if (ov < tot[q]) {
        jv = q;
        got = true;
      } else {
        ov -= tot[q];
      }
    }
  }
  int cj = 0;
#pragma unroll
  for (int q = 0; q < NB; ++q) cj = q == jv ? cnt[q] : cj;
  const int cscan = wave_scan(cj);
  const uint64_t m = __builtin_amdgcn_ballot_w64(cscan > ov);
  if (m == 0) return false;  // not reached: ov < tot[jv], the bucket's total
  const int sel = __builtin_ctzll(m);
  int off = ov - __builtin_amdgcn_readlane(cscan - cj, sel);
  int ubase = __builtin_amdgcn_readlane(uscan - usum, sel);
  bool found = false;
  int jsel = 0, nrb = 1, nf = 0;
#pragma unroll
  for (int j = 0; j < kExactPerLane; ++j) {
    const int r = __builtin_amdgcn_readlane(rbs[j], sel);
    const int f = __builtin_amdgcn_readlane(nfull[j], sel);
    const int pb = __builtin_amdgcn_readlane(pbk[j], sel);
    const int c = jv == NB - 1 ? f * r : (pb == jv ? r : 0);
    if (!found) {
      if (off < c) {
        found = true;
        jsel = j;
        nrb = r;
        nf = f;
      } else {
        off -= c;
        ubase += r;
      }
    }
  }
  int L = 0, c0 = 0, c1 = 0, co = -1;
#pragma unroll
  for (int j = 0; j < kExactPerLane; ++j) {
    if (j == jsel) {
      L = __builtin_amdgcn_readlane(Lq[j], sel);
      c0 = __builtin_amdgcn_readlane(c0q[j], sel);
      c1 = __builtin_amdgcn_readlane(c1q[j], sel);
      co = __builtin_amdgcn_readlane(coq[j], sel);
    }
  }
  w.b = sel * k + jsel;
  if (jv == NB - 1) {
    w.s = off / nrb;
    w.rg = off - w.s * nrb;
  } else {  // the sequence's partial split
    w.s = nf;
    w.rg = off;
  }
  w.hg = slot - kk * a.inner;
  w.unit = (ubase + w.rg) * a.inner + w.hg;
  w.L = L;
  w.sr = seq_rows_of<CAUSAL>(a, w.b, L, c0, c1, co);
  return true;
}

// The schedule of a workgroup.  Exact (above) when a.exact; otherwise one
// block per (sequence, split) pair and unit slot (kv-head group, row block),
// the pairs in split-major order (decode_pair), whose empty blocks exit.
// XCD-aware: blocks x, x + 8, ... run on one XCD.  With 8 pairs or more,
// pair p runs on XCD p mod 8 with all its unit slots back to back; with
// fewer (a prefill-shaped call: few sequences, many row blocks) XCD x takes
// the x-th eighth of the (pair, slot) list, so every XCD has work.  False:
// no work.
//
// On the per-block schedule the sequence's length (and, for a varlen batch,
// its token offsets) is read here but used by the kernels only after they
// have issued the loads of their q rows and first page-table window, which do
// not depend on it for fixed-length batches: the loads then share one memory
// round trip.
template <bool CAUSAL>
__device__ __forceinline__ bool work_of(const DecodeArgs &a, Work &w) {
  const int x = blockIdx.x;
  const int xcd = x & 7;
  const int slot = x >> 3;
  if (a.exact) return a.lpt ? work_lpt<CAUSAL>(a, xcd, slot, w) : work_exact<CAUSAL>(a, xcd, slot, w);
  int inner_idx, outer_idx;
  if (a.outer >= 8) {
    inner_idx = slot % a.inner;
    outer_idx = (slot / a.inner) * 8 + xcd;
    if (outer_idx >= a.outer) return false;
  } else {
    const int total = a.outer * a.inner;
    const int per = (total + 7) >> 3;
    const int i = xcd * per + slot;
    if (slot >= per || i >= total) return false;
    outer_idx = i / a.inner;
    inner_idx = i - outer_idx * a.inner;
  }
  decode_pair(outer_idx, a.B, w.b, w.s);
  w.hg = inner_idx / a.nrb;
  w.rg = inner_idx - w.hg * a.nrb;
  w.unit = w.b * a.inner + inner_idx;
  w.L = a.kv_lens[w.b];
  w.sr = seq_rows<CAUSAL>(a, w.b, w.L);
  return true;
}

// Output row (token, query head) of packed row rr (= i * G + k) of kv head g
// of the sequence whose first token is tok0.
__device__ __forceinline__ int64_t out_row(const DecodeArgs &a, int64_t tok0, int g, int rr) {
  const int i = rr / a.G;
  const int h = g * a.G + (rr - i * a.G);
  return (tok0 + i) * a.Hq + h;
}

// Head pairing (a.pair): kv heads 2g and 2g + 1 of D/2 columns each, adjacent
// in every key row, are read as one head g of D columns, and its G = 2 G'
// packed rows per token are the query heads of both.  Packed row rr belongs
// to the second of the two (its q fills columns D/2 .. D-1, zeros elsewhere,
// and its output is those columns) when its query head is among the last G'
// of the group.  Its scores are those of its own head, since the other half
// of q is zero.
__device__ __forceinline__ int pair_half(const DecodeArgs &a, int rr) {
  return (rr - (rr / a.G) * a.G) >= (a.G >> 1) ? 1 : 0;
}

// ---- log-sum-exp merge of split partials -----------------------------------
// For each of `nrows` rows (row index rowf(r); partials of a row S apart) and
// each 4-element group of its D outputs, one thread walks the first nsp <= S
// partials in split order with
// an online merge: partials with l_s = 0 are skipped (their o rows are never
// used); otherwise, when m_s exceeds the running max M the running sums are
// rescaled by exp(M - m_s), then w_s = l_s exp(m_s - M) is added to W and
// w_s o_s to the accumulator.  out = acc * (1 / W), 0 when W = 0, and o_s
// itself when s is the only partial with l_s > 0 (so a row that one split
// covers gets the same bits whether that split wrote the output or a merge
// of its partial did).  This is
// the log-sum-exp rule M = max m_s, out = sum_s l_s e^(m_s - M) o_s / sum_s
// l_s e^(m_s - M), evaluated in one pass.  Each thread loads the (m, l) of
// the splits itself, so no LDS and no barrier are needed.  Both the in-kernel
// merge and the combine kernel run this code, so their results are
// bit-identical.  Run by nthreads threads (any number); rowf must be cheap
// (it is evaluated once per group).  DEV: the partials were written by other
// workgroups of the running launch.
constexpr int kMergeBatch = 16;  // partials in flight per thread

template <bool DEV>
__device__ __forceinline__ float4 load4(const float *p) {  // p 16-byte aligned
  if constexpr (DEV) {
    const float2 lo = load2<true>(p);
    const float2 hi = load2<true>(p + 2);
    return make_float4(lo.x, lo.y, hi.x, hi.y);
  } else {
    return *reinterpret_cast<const float4 *>(p);
  }
}

template <int D, bool DEV, class RowF>
__device__ void merge_rows(const float *o_part, const float *ml_part, int S, int nsp, RowF rowf, int nrows,
                           uint16_t *out, float *out_f32, int nthreads) {
  constexpr int DQ = D / 4;  // 4-element groups per row (a power of two)
  constexpr int NB = kMergeBatch;
  const int tid = threadIdx.x;
  // this thread's groups: tid, tid + nthreads, ...; its items: (group,
  // split) pairs, group-major, split order within a group
  const int ngroups = nrows * DQ;
  const int mine = tid < ngroups ? (ngroups - 1 - tid) / nthreads + 1 : 0;
  const int items = mine * nsp;
  float4 ov[NB];
  float2 mv[NB];
  int ig = tid, isp = 0;
  const float *ip = o_part, *im = ml_part;
  auto group_start = [&](int gidx) {
    const int r = gidx / DQ;
    const int64_t row = rowf(r);
    ip = o_part + row * S * D + 4 * (gidx - r * DQ);
    im = ml_part + row * S * 2;
  };
  if (items > 0) group_start(ig);
  auto issue = [&](int i0) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      if (i0 + k < items) {
        ov[k] = load4<DEV>(ip);
        mv[k] = load2<DEV>(im);
        if (++isp == nsp) {
          isp = 0;
          ig += nthreads;
          if (i0 + k + 1 < items) group_start(ig);
        } else {
          ip += D;
          im += 2;
        }
      }
    }
  };
  issue(0);

  float M = -INFINITY, W = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 first = acc;  // o of the first partial with l > 0
  int used = 0;        // partials with l > 0 so far
  int cg = tid, csp = 0;
  for (int i0 = 0; i0 < items; i0 += NB) {
    if (i0 > 0) issue(i0);
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      if (i0 + k < items) {
        const float m = mv[k].x;
        const float l = mv[k].y;
        if (l > 0.f) {
          if (used++ == 0) first = ov[k];
          if (m > M) {
            const float sc = fast_exp2((M - m) * kLog2e);
            W *= sc;
            acc.x *= sc;
            acc.y *= sc;
            acc.z *= sc;
            acc.w *= sc;
            M = m;
          }
          const float wk = l * fast_exp2((m - M) * kLog2e);
          W += wk;
          acc.x = fmaf(wk, ov[k].x, acc.x);
          acc.y = fmaf(wk, ov[k].y, acc.y);
          acc.z = fmaf(wk, ov[k].z, acc.z);
          acc.w = fmaf(wk, ov[k].w, acc.w);
        }
        if (++csp == nsp) {
          const int r = cg / DQ;
          const int64_t row = rowf(r);
          const int d = 4 * (cg - r * DQ);
          const float inv = W > 0.f ? 1.f / W : 0.f;
          const float4 res =
              used == 1 ? first : make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
          const uint32_t lo = (uint32_t)f32_to_bf16_rne(res.x) | ((uint32_t)f32_to_bf16_rne(res.y) << 16);
          const uint32_t hi = (uint32_t)f32_to_bf16_rne(res.z) | ((uint32_t)f32_to_bf16_rne(res.w) << 16);
          *reinterpret_cast<uint2 *>(out + row * D + d) = make_uint2(lo, hi);
          if (out_f32) *reinterpret_cast<float4 *>(out_f32 + row * D + d) = res;
          M = -INFINITY;
          W = 0.f;
          acc = make_float4(0.f, 0.f, 0.f, 0.f);
          used = 0;
          csp = 0;
          cg += nthreads;
        }
      }
    }
  }
}

// A split with no keys of its unit, outside the in-kernel merge: its (m, l)
// entries become (-inf, 0) (its o_part rows are left untouched, never read).
// Block row ri = r * hpb + hh is packed row r0 + r of kv head hg * hpb + hh.
__device__ __forceinline__ void empty_partials(const DecodeArgs &a, int64_t tok0, int hg, int r0, int s, int nrows) {
  for (int ri = threadIdx.x; ri < nrows; ri += blockDim.x) {
    const int64_t row = out_row(a, tok0, hg * a.hpb + (ri & (a.hpb - 1)), r0 + (ri >> a.lhpb));
    *reinterpret_cast<float2 *>(a.ml_part + (row * a.S + s) * 2) = make_float2(-INFINITY, 0.f);
  }
}

// Epilogue shared by the split kernels once a block's waves have left their
// results in LDS, for its nrows output rows: `rowtab[r]` is the output row of
// block row r; `item(r, d, M, W, v)` gives the row's base-2 reference max M,
// its total weight W and the normalised results at columns d .. d + 7 (0 when
// the row saw no key).  `direct`: write the output (the unit's only split
// with keys).  Otherwise write this split's partial (o, m in natural-log
// units, l = W); an empty split (W = 0) writes only (m, l) = (-inf, 0).
// Eight columns per item: the output goes out in 16-byte stores, which keeps
// the store count low while other workgroups of the CU stream K/V.
template <int D, class ItemF>
__device__ void write_rows(const DecodeArgs &a, int s, bool direct, const int64_t *rowtab, int nrows, ItemF item,
                           int nthreads) {
  constexpr int DG = D / 8;
  for (int idx = threadIdx.x; idx < nrows * DG; idx += nthreads) {
    const int r = idx / DG;
    const int d = 8 * (idx - r * DG);
    const int64_t row = rowtab[r];
    float M, W, v[8];
    item(r, d, M, W, v);
    if (direct) {
      uint4 pk;
      pk.x = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
      pk.y = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
      pk.z = (uint32_t)f32_to_bf16_rne(v[4]) | ((uint32_t)f32_to_bf16_rne(v[5]) << 16);
      pk.w = (uint32_t)f32_to_bf16_rne(v[6]) | ((uint32_t)f32_to_bf16_rne(v[7]) << 16);
      *reinterpret_cast<uint4 *>(a.out + row * D + d) = pk;
      if (a.out_f32) {
        float4 *o32 = reinterpret_cast<float4 *>(a.out_f32 + row * D + d);
        o32[0] = make_float4(v[0], v[1], v[2], v[3]);
        o32[1] = make_float4(v[4], v[5], v[6], v[7]);
      }
    } else {
      float *po = a.o_part + (row * a.S + s) * D + d;
      float *pm = a.ml_part + (row * a.S + s) * 2;
      const float mx = W > 0.f ? M * kLn2 : -INFINITY;
      if (a.fused) {  // merged by another workgroup of this launch
        if (W > 0.f) {
          store_part4(a, po, v[0], v[1], v[2], v[3]);
          store_part4(a, po + 4, v[4], v[5], v[6], v[7]);
        }
        if (d == 0) store_dev2(pm, mx, W);
      } else {        // read after this kernel has ended
        if (W > 0.f) {
          reinterpret_cast<float4 *>(po)[0] = make_float4(v[0], v[1], v[2], v[3]);
          reinterpret_cast<float4 *>(po)[1] = make_float4(v[4], v[5], v[6], v[7]);
        }
        if (d == 0) *reinterpret_cast<float2 *>(pm) = make_float2(mx, W);
      }
    }
  }
}

// Wave merge factors of one row: from the NW waves' (m, l) (base-2 m), the
// row's reference max M, total weight W and each wave's normalised factor
// exp2(m_w - M) / W (0 for waves that saw no key, all 0 when W = 0).
template <int NW>
__device__ __forceinline__ void wave_factors(const float (&m)[NW], const float (&l)[NW], float &M, float &W,
                                             float (&f)[NW]) {
  M = -INFINITY;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww)
    if (l[ww] > 0.f) M = fmaxf(M, m[ww]);
  W = 0.f;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) {
    f[ww] = (l[ww] > 0.f) ? fast_exp2(m[ww] - M) : 0.f;
    W = fmaf(f[ww], l[ww], W);
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) f[ww] *= inv;
}

// Where column group c (4 floats) of a merge-buffer row is kept, in 16-byte
// units, when the columns are swizzled: groups 16..31 of each 32 swap
// neighbours, so that the 16 lanes of one LDS pass that read groups 0, 2,
// .., 30 (or 1, 3, .., 31) of a 128-column row hit 16 distinct bank groups (a
// pass covers 256 bytes of banks).
template <bool SWZ>
__device__ __forceinline__ int ob_unit(int c) { return SWZ ? c ^ ((c >> 4) & 1) : c; }

// The merged result of a block row at columns d .. d + 7 from the per-wave
// results in LDS: wave slot kk*HR + rs (rs: the row's slot within a wave's
// block of HR rows) holds wave kk's (m, l) in mlb and its unnormalised O row
// in ob (row stride OBS floats, column groups placed by ob_unit<SWZ>, d a
// multiple of 8 and rows 16-byte aligned); waves kk >= wph hold no row of
// this head.  All loads are issued together, from clamped slots, and unused
// waves are masked after loading, so no branch separates them.
template <int NW, int OBS, bool SWZ = false>
__device__ __forceinline__ void merge_waves(const float *mlb, const float *ob, int HR, int wph, int rs, int d,
                                            float &M, float &W, float (&v)[8]) {
  float mw[NW], lw[NW], f[NW];
  float4 o0[NW], o1[NW];
#pragma unroll
  for (int kk = 0; kk < NW; ++kk) {
    const int slot = (kk < wph ? kk : wph - 1) * HR + rs;
    const float2 ml = *reinterpret_cast<const float2 *>(mlb + 2 * slot);
    if constexpr (SWZ) {
      const float4 *orow = reinterpret_cast<const float4 *>(ob + slot * OBS);
      o0[kk] = orow[ob_unit<true>(d / 4)];
      o1[kk] = orow[ob_unit<true>(d / 4 + 1)];
    } else {
      const float4 *orow = reinterpret_cast<const float4 *>(ob + slot * OBS + d);
      o0[kk] = orow[0];
      o1[kk] = orow[1];
    }
    mw[kk] = kk < wph ? ml.x : -INFINITY;
    lw[kk] = kk < wph ? ml.y : 0.f;
  }
  wave_factors<NW>(mw, lw, M, W, f);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = 0.f;
#pragma unroll
  for (int kk = 0; kk < NW; ++kk) {   // f = 0 for unused waves (their loads are finite rows of wave wph - 1)
    v[0] = fmaf(f[kk], o0[kk].x, v[0]);
    v[1] = fmaf(f[kk], o0[kk].y, v[1]);
    v[2] = fmaf(f[kk], o0[kk].z, v[2]);
    v[3] = fmaf(f[kk], o0[kk].w, v[3]);
    v[4] = fmaf(f[kk], o1[kk].x, v[4]);
    v[5] = fmaf(f[kk], o1[kk].y, v[5]);
    v[6] = fmaf(f[kk], o1[kk].z, v[6]);
    v[7] = fmaf(f[kk], o1[kk].w, v[7]);
  }
}

// With a.fused (several splits, one call): each of the unit's n active
// splits (those that hold keys of it) stores its partial, waits for those
// stores to complete and counts itself in; the block that arrives last merges
// the n partials and resets the counter, so the workspace is ready for the
// next call.  `lds` (one int) is free: all block threads are past their last
// use of it when this is called.
template <int D>
__device__ void fused_tail(const DecodeArgs &a, int unit, int n, const int64_t *rowtab, int nrows, float *lds,
                           int nthreads) {
  __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores have completed
  __syncthreads();
  int *flag = reinterpret_cast<int *>(lds);
  if (threadIdx.x == 0) flag[0] = atomicAdd(a.counters + unit, 1) == n - 1;
  __syncthreads();
  const bool last = flag[0] != 0;
  __syncthreads();
  if (!last) return;
  merge_rows<D, true>(a.o_part, a.ml_part, a.S, n, [&](int r) { return rowtab[r]; }, nrows, a.out, a.out_f32,
                      nthreads);
  if (threadIdx.x == 0) a.counters[unit] = 0;  // ready for the next call
}

}  // namespace dev
}  // namespace pkv
