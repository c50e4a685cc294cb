// pkv_decode.hip -- split-KV paged decode kernel for CDNA4 (gfx950), VALU path.
//
// Method (AstrAI commit d565d44, "csrc/kernels/attn_paged_decode.cu", commit
// notes on the scalar split-KV paged decode kernel and the MMA variant): every
// workgroup takes one key split s of one (sequence b, kv-head group, row
// block) unit; the group holds hpb kv heads (1, 2 or 4).  The query rows that
// share kv head g (G query heads x q_len tokens: "GQA head packing") are
// processed together, so every K/V byte is read from HBM once per split.  Keys are resolved through the page table, scores are accumulated
// with an online softmax (running max m and sum l per row), and the split
// leaves either the final output (one split) or a normalised partial plus
// (m, l) for the combine kernel.
//
// gfx950 mapping:
//  * a workgroup is kWavesPerBlock wave64s; wave w works on kv head
//    w % hpb of the group and, with the other NW / hpb waves of that head,
//    takes every (NW / hpb)-th tile of T keys, keeping its own (m, l, acc);
//    the waves of a head merge once at the end through LDS, so the key loop
//    has no workgroup barrier.  With several heads per workgroup its waves
//    read the neighbouring head slices of the same page slots at about the
//    same time, which suits HBM better than one head's short slices alone;
//  * the split's slice of the page table is staged in LDS once (in windows of
//    kBtCap pages), so a K/V address costs an LDS read, not an HBM round trip;
//  * K/V tiles are double-buffered in registers: the loads of a wave's next
//    tile are in flight while it computes the current one;
//  * QK^T uses v_dot2_f32_bf16 on packed bf16 pairs (exact products, fp32
//    accumulation) in a "key-major" lane layout: D/32 lanes per key, each
//    holding 32 elements of q and k, summed across those lanes with DPP;
//  * PV uses fp32 FMAs in a "d-major" layout: D/8 lanes per key, each owning
//    8 output columns; probabilities cross between the two layouts through a
//    per-wave LDS slice (no barrier: LDS is in order within a wave);
//  * cross-lane max/sum use DPP (quad_perm, row mirrors, row_ror) and the
//    gfx950 permlane16/32 swaps, no LDS traffic;
//  * K and V rows are fetched with 128-bit loads; rows past the split end are
//    never loaded (tails read as zero);
//  * the workgroup index is decoded so that the head-group x row-block
//    siblings of a (b, s) pair land on the same XCD back to back (blocks are
//    dealt to the 8 XCDs round-robin), so they share that XCD's L2 for the
//    interleaved kv heads of a page slot;
//  * scores live in base 2 (scale * log2 e folded in) and use v_exp_f32;
//    exclusion (tail, causal, -inf mask) is a select, never an add.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

int rows_per_block(int R, int head_dim, int hpb) {
  switch (kernel_kind(R, head_dim, hpb)) {
    case kKernelPrefill: return kPrefillRows;
    case kKernelValu: return R <= 1 ? 1 : R <= 2 ? 2 : 4;   // 4: head_dim 256 only (use_mfma)
    default: return R <= 16 ? 16 : 32;
  }
}

// Keys per VALU wave tile (one QK pass: 64 / (D/32)), never below the
// 16-key tile of the matrix-core kernel, so split boundaries suit both.
int tile_keys(int head_dim) {
  const int t = 64 / (head_dim / 32);
  return t < 16 ? 16 : t;
}

namespace {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

using namespace dev;

constexpr int kBtCap = 1024;            // page-table entries staged in LDS per window
constexpr float kRescaleLog2 = 8.f;     // lazy-rescale threshold (base-2 score units)

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}
__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

constexpr int ilog2c(int x) { return x <= 1 ? 0 : 1 + ilog2c(x / 2); }

// Reduce over lane bits [0, HI) (HI <= 3) of independent values.
template <int HI, class Op>
__device__ __forceinline__ float reduce_lo(float x) {
  if constexpr (HI >= 1) x = Op::f(x, dpp<kXor1>(x));
  if constexpr (HI >= 2) x = Op::f(x, dpp<kXor2>(x));
  if constexpr (HI >= 3) x = Op::f(x, dpp<kHalfMirror>(x));  // quads already reduced
  return x;
}

// Reduce over lane bits [LO, 6) when lanes that differ only in bits [0, LO)
// already hold equal values (mirror pairings are then valid).
template <int LO, class Op>
__device__ __forceinline__ float reduce_hi_grouped(float x) {
  if constexpr (LO <= 0) x = Op::f(x, dpp<kXor1>(x));
  if constexpr (LO <= 1) x = Op::f(x, dpp<kXor2>(x));
  if constexpr (LO <= 2) x = Op::f(x, dpp<kHalfMirror>(x));
  if constexpr (LO <= 3) x = Op::f(x, dpp<kMirror>(x));
  if constexpr (LO <= 4) x = xor16<Op>(x);
  x = xor32<Op>(x);
  return x;
}

__device__ __forceinline__ uint32_t comp(const uint4 &v, int e) {
  return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}

template <int D, int RP>
struct Layout {
  static constexpr int NW = kWavesPerBlock;
  static constexpr int LPK = D / 32;       // lanes per key, QK layout
  static constexpr int KPP = 64 / LPK;     // keys per QK pass
  static constexpr int NPASS = 1;
  static constexpr int T = KPP * NPASS;    // keys per wave tile
  static constexpr int LPV = D / 8;        // lanes per key, PV layout
  static constexpr int KPV = 64 / LPV;     // keys per PV step
  static constexpr int NSTEP = T / KPV;    // PV steps per tile
  static constexpr int LOG_LPK = ilog2c(LPK);
  static constexpr int LOG_LPV = ilog2c(LPV);
  static constexpr int PBUF = NW * T * RP;             // floats
  static constexpr int KBUF = NW * T * D / 2;          // per-wave K tile (bf16 pairs, as floats)
  // XOR swizzle of a K row's 16-byte chunks in the per-wave K tile, so the
  // key-major reads (lane = key jq, part qq) hit distinct LDS banks
  static constexpr int SW_MUL = LPK;
  static constexpr int SW_SHIFT = LPK >= 4 ? 0 : (LPK == 2 ? 1 : 2);
  static constexpr int SW_MASK = LPK >= 8 ? 1 : 3;
  __device__ static int kslot(int ch, int row) { return ch ^ (SW_MUL * ((row >> SW_SHIFT) & SW_MASK)); }
  // merge phase: per-wave O rows and (m, l)
  static constexpr int MERGE = NW * RP * D + NW * RP * 2;
  static constexpr int MAIN = kBtCap + 4 + PBUF + KBUF;  // page-table slice (+1 page when a window
                                                         // starts mid-page), p and K slices
  static constexpr int SMEM = MAIN > MERGE ? MAIN : MERGE;
};

// Per-wave context of the split kernel.
template <int D, int RP>
struct Ctx {
  const uint16_t *kbase, *vbase;
  const int *bt;         // LDS page-table slice
  int p0;                // first page of the slice
  int page_shift, pmask;
  int64_t page_stride;
  int row_stride;
  int kb;                // first key of the split
  int ke;                // end of the keys this block may see
  int R;                 // packed rows of the sequence per kv head
  int jq, qq, kg, ds;
};

template <int D, int RP, bool MASK>
struct Tile {
  uint4 k[Layout<D, RP>::NSTEP];   // K rows in the row layout (same rows/chunks as v)
  uint4 v[Layout<D, RP>::NSTEP];
  float mk[MASK ? Layout<D, RP>::NPASS : 1][MASK ? RP : 1];  // additive mask (log2 units) of this lane's key
};

template <int D, int RP>
__device__ __forceinline__ int64_t row_offset(const Ctx<D, RP> &c, int j) {
  const int page = c.bt[(j >> c.page_shift) - c.p0];
  return (int64_t)page * c.page_stride + (int64_t)(j & c.pmask) * c.row_stride;
}

// Issue the loads of tile `base` (keys base .. base+T-1) into registers.
// K and V use the same row layout: lane (kg, ds) fetches 16 bytes (chunk ds)
// of rows base + st*KPV + kg, so each wave instruction reads whole rows and
// one page lookup serves both caches.  Rows past the end are clamped to the
// last valid key: they load finite data that the score mask gives zero
// weight, so no lane branches and no register is zero-filled.  With UPAGE (a
// page holds at least one tile) the tile's page is wave-uniform and resolved
// once, in scalar registers.
template <int D, int RP, bool MASK, bool UPAGE>
__device__ __forceinline__ void load_tile(const DecodeArgs &a, const Ctx<D, RP> &c, int b, int r0, int base,
                                          Tile<D, RP, MASK> &t) {
  using Lay = Layout<D, RP>;
  const int jlast = c.ke - 1;
  if constexpr (MASK) {
#pragma unroll
    for (int pp = 0; pp < Lay::NPASS; ++pp) {
      int j = base + pp * Lay::KPP + c.jq;
      j = j < jlast ? j : jlast;
      const float *mrow = a.mask + (int64_t)b * a.mask_sb + j;
      // one load per row on every path (a 2D mask, mask_sq = 0, loads the same
      // entry for each row): a load count that depends on a runtime branch
      // would make the compiler wait for all loads at the loop header
#pragma unroll
      for (int r = 0; r < RP; ++r) {
        const int rr = r0 + r < c.R ? r0 + r : c.R - 1;
        t.mk[pp][r] = mrow[(int64_t)(rr / a.G) * a.mask_sq];
      }
    }
  }
  if constexpr (UPAGE) {
    // a tile past the window end (an unconditional prefetch) reads the last key's page
    const int bj = base < jlast ? base : jlast;
    const int page = __builtin_amdgcn_readfirstlane(c.bt[(bj >> c.page_shift) - c.p0]);
    // the tile's first key in the scalar offset; keys j of the tile are j - bj < T rows further
    const int64_t pofs = (int64_t)page * c.page_stride + (int64_t)(bj & c.pmask) * c.row_stride;
    const uint16_t *kp = c.kbase + pofs;
    const uint16_t *vp = c.vbase + pofs;
    if (D == 256 && base + Lay::T - 1 <= jlast) {
      // every key of the tile exists (bj = base): one multiply for the lane,
      // a wave-uniform step per load (at D = 256 only: 16 x 4096 keys, one
      // query head per kv head, 85.0 -> 83.9 us; at D = 64 and 128 the same
      // shapes ran 5% slower, at D = 32 no change)
      const uint32_t o0 = (uint32_t)(c.kg * c.row_stride);
      const uint32_t step = (uint32_t)(Lay::KPV * c.row_stride);
#pragma unroll
      for (int st = 0; st < Lay::NSTEP; ++st) {
        const uint32_t off = o0 + st * step;
        t.k[st] = load_stream(reinterpret_cast<const uint4 *>(kp + off) + c.ds);
        t.v[st] = load_stream(reinterpret_cast<const uint4 *>(vp + off) + c.ds);
      }
    } else {
#pragma unroll
      for (int st = 0; st < Lay::NSTEP; ++st) {
        int j = base + st * Lay::KPV + c.kg;
        j = j < jlast ? j : jlast;
        const uint32_t off = (uint32_t)((j - bj) * c.row_stride);
        t.k[st] = load_stream(reinterpret_cast<const uint4 *>(kp + off) + c.ds);
        t.v[st] = load_stream(reinterpret_cast<const uint4 *>(vp + off) + c.ds);
      }
    }
  } else {
#pragma unroll
    for (int st = 0; st < Lay::NSTEP; ++st) {
      int j = base + st * Lay::KPV + c.kg;
      j = j < jlast ? j : jlast;
      const int64_t off = row_offset(c, j);
      t.k[st] = load_stream(reinterpret_cast<const uint4 *>(c.kbase + off) + c.ds);
      t.v[st] = load_stream(reinterpret_cast<const uint4 *>(c.vbase + off) + c.ds);
    }
  }
}

// Online-softmax state of one wave.
template <int RP>
struct State {
  float m[RP];        // running max (base-2 units), uniform across the wave
  float l[RP];        // running sum of this lane's key group (QK layout)
  float acc[RP][8];   // PV accumulator, this lane's 8 columns and key group
};

// q rows of a wave, in registers: this lane's chunks qq + LPK*c4 of every row
template <int D, int RP>
struct QRows {
  uint4 v[RP][4];
  __device__ __forceinline__ uint4 get(int r, int c4, int) const { return v[r][c4]; }
};

template <int D, int RP, bool CAUSAL, bool MASK, class Q>
__device__ __forceinline__ void compute_tile(const DecodeArgs &a, const Ctx<D, RP> &c, int base,
                                             const Tile<D, RP, MASK> &t, const Q &qrows,
                                             const int (&lim)[RP], float *pbuf, float *kbuf, State<RP> &st) {
  using Lay = Layout<D, RP>;
  constexpr int NPASS = Lay::NPASS, KPP = Lay::KPP, LPK = Lay::LPK;
  // K tile: row layout (registers) -> per-wave LDS slice -> key-major layout
  {
    uint4 *kw = reinterpret_cast<uint4 *>(kbuf);
#pragma unroll
    for (int st = 0; st < Lay::NSTEP; ++st) {
      const int row = st * Lay::KPV + c.kg;
      kw[row * (D / 8) + Lay::kslot(c.ds, row)] = t.k[st];
    }
  }
  __builtin_amdgcn_wave_barrier();
  // scores, summed over the LPK lanes of each key
  float sc[NPASS][RP];
#pragma unroll
  for (int pp = 0; pp < NPASS; ++pp) {
    float d[RP];
#pragma unroll
    for (int r = 0; r < RP; ++r) d[r] = 0.f;
    const int krow = pp * KPP + c.jq;
    const uint4 *kr = reinterpret_cast<const uint4 *>(kbuf) + krow * (D / 8);
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const uint4 kk = kr[Lay::kslot(c.qq + LPK * c4, krow)];
#pragma unroll
      for (int r = 0; r < RP; ++r) {
        const uint4 qv = qrows.get(r, c4, c.qq);
        d[r] = dot2_bf16(kk.x, qv.x, d[r]);
        d[r] = dot2_bf16(kk.y, qv.y, d[r]);
        d[r] = dot2_bf16(kk.z, qv.z, d[r]);
        d[r] = dot2_bf16(kk.w, qv.w, d[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < RP; ++r) sc[pp][r] = reduce_lo<Lay::LOG_LPK, OpSum>(d[r]);
  }
  // scale, mask, visibility
#pragma unroll
  for (int pp = 0; pp < NPASS; ++pp) {
    const int j = base + pp * KPP + c.jq;
    const bool in = j < c.ke;
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      const float v = MASK ? fmaf(sc[pp][r], a.scale_log2, t.mk[pp][r] * kLog2e) : sc[pp][r] * a.scale_log2;
      const bool vis = CAUSAL ? (in && j < lim[r]) : (in && lim[r] > 0);
      sc[pp][r] = vis ? v : -INFINITY;
    }
  }
  // online softmax with a lazy reference: the running reference m only moves
  // (and the accumulators are rescaled) when a score exceeds it by more than
  // kRescaleLog2; otherwise p = 2^(s - m) <= 2^kRescaleLog2, which fp32 holds
  // with room to spare.  m is uniform across the wave, so the branch is too.
  float dmax = -INFINITY;   // NaN (-inf - -inf) is ignored by fmaxf
#pragma unroll
  for (int r = 0; r < RP; ++r)
#pragma unroll
    for (int pp = 0; pp < NPASS; ++pp) dmax = fmaxf(dmax, sc[pp][r] - st.m[r]);
  const bool above = dmax > kRescaleLog2;
  if (__builtin_amdgcn_ballot_w64(above) != 0) {
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      float mt = sc[0][r];
#pragma unroll
      for (int pp = 1; pp < NPASS; ++pp) mt = fmaxf(mt, sc[pp][r]);
      mt = reduce_hi_grouped<Lay::LOG_LPK, OpMax>(mt);
      const float mnew = fmaxf(st.m[r], mt);
      const float alpha = mnew == -INFINITY ? 1.f : fast_exp2(st.m[r] - mnew);
      st.m[r] = mnew;
      st.l[r] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) st.acc[r][e] *= alpha;
    }
  }
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    const float use = st.m[r] == -INFINITY ? 0.f : st.m[r];
    float lsum = 0.f;
#pragma unroll
    for (int pp = 0; pp < NPASS; ++pp) {
      const float pv = fast_exp2(sc[pp][r] - use);
      lsum += pv;
      pbuf[(pp * KPP + c.jq) * RP + r] = pv;   // the LPK lanes of a key store the same value
    }
    st.l[r] += lsum;
  }
  __builtin_amdgcn_wave_barrier();

  // PV
#pragma unroll
  for (int s2 = 0; s2 < Lay::NSTEP; ++s2) {
    const int key = s2 * Lay::KPV + c.kg;
    float pr[RP];
    if constexpr (RP >= 4) {
#pragma unroll
      for (int r4 = 0; r4 < RP / 4; ++r4) {
        const float4 t4 = reinterpret_cast<const float4 *>(pbuf + key * RP)[r4];
        pr[4 * r4 + 0] = t4.x;
        pr[4 * r4 + 1] = t4.y;
        pr[4 * r4 + 2] = t4.z;
        pr[4 * r4 + 3] = t4.w;
      }
    } else if constexpr (RP == 2) {
      const float2 t2 = reinterpret_cast<const float2 *>(pbuf + key * RP)[0];
      pr[0] = t2.x;
      pr[1] = t2.y;
    } else {
      pr[0] = pbuf[key];
    }
    float vf[8];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const uint32_t u = comp(t.v[s2], e2);
      vf[2 * e2] = bf16_lo(u);
      vf[2 * e2 + 1] = bf16_hi(u);
    }
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) st.acc[r][e] = fmaf(pr[r], vf[e], st.acc[r][e]);
  }
  __builtin_amdgcn_wave_barrier();
}

// Register tiles per wave in the key loop (see tile_loop).
template <int D, int RP>
constexpr int valu_nbuf() { return 2; }

// The key-tile loop of one wave (tiles t0, t0 + tstep, ... < ntiles), NBUF
// register tiles in a ring: while tile i computes, the loads of tiles i+1 ..
// i+NBUF-1 are in flight; after it, its registers take the loads of tile
// i+NBUF.  Whole rounds run while every prefetch of the round is a tile of
// this wave: their loads are issued unconditionally and in a fixed order, and
// a round has no early exit, so the number of loads in flight is the same on
// both paths into the loop header (a conditional load or an exit there makes
// the compiler wait for all loads).  The last tiles are computed after the
// loop with prefetches only of tiles that exist, so no load is left in flight
// past the last tile (the epilogue would wait for it before reusing its
// registers).  With fewer tiles than NBUF the first loads repeat the last key
// (clamped in load_tile).
template <int D, int RP, bool CAUSAL, bool MASK, bool UPAGE, class Q, int NBUF = valu_nbuf<D, RP>()>
__device__ __forceinline__ void tile_loop(const DecodeArgs &a, const Ctx<D, RP> &c, int b, int r0, int wb,
                                          int t0, int tstep, int ntiles, const Q &qrows, const int (&lim)[RP],
                                          float *pbuf, float *kbuf, State<RP> &st) {
  using Lay = Layout<D, RP>;
  constexpr int T = Lay::T;
  if (t0 >= ntiles) return;
  Tile<D, RP, MASK> tr[NBUF];
#pragma unroll
  for (int i = 0; i < NBUF; ++i) {
    load_tile<D, RP, MASK, UPAGE>(a, c, b, r0, wb + (t0 + i * tstep) * T, tr[i]);
    __builtin_amdgcn_sched_barrier(0);
  }
  int t = t0;
  for (; t + (2 * NBUF - 1) * tstep < ntiles; t += NBUF * tstep) {
#pragma unroll
    for (int i = 0; i < NBUF; ++i) {
      compute_tile<D, RP, CAUSAL, MASK>(a, c, wb + (t + i * tstep) * T, tr[i], qrows, lim, pbuf, kbuf, st);
      load_tile<D, RP, MASK, UPAGE>(a, c, b, r0, wb + (t + (i + NBUF) * tstep) * T, tr[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int i = 0; i < NBUF; ++i) {
    const int tt = t + i * tstep;
    if (tt < ntiles) {   // wave-uniform
      compute_tile<D, RP, CAUSAL, MASK>(a, c, wb + tt * T, tr[i], qrows, lim, pbuf, kbuf, st);
      if (tt + NBUF * tstep < ntiles) load_tile<D, RP, MASK, UPAGE>(a, c, b, r0, wb + (tt + NBUF * tstep) * T, tr[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < NBUF; ++i) {
    const int tt = t + (NBUF + i) * tstep;
    if (tt < ntiles) compute_tile<D, RP, CAUSAL, MASK>(a, c, wb + tt * T, tr[i], qrows, lim, pbuf, kbuf, st);
  }
}

// PAIR: head pairing (pair_half), two kv heads of D/2 columns per head of the
// launch; q, the output and the partials have DO = D/2 columns.
template <int D, int RP, bool CAUSAL, bool MASK, bool UPAGE, bool PAIR = false>
__global__ __launch_bounds__(kWavesPerBlock * 64) void split_decode_valu(const DecodeArgs a) {
  using Lay = Layout<D, RP>;
  constexpr int NW = Lay::NW, LPK = Lay::LPK, T = Lay::T, LPV = Lay::LPV;
  constexpr int DO = PAIR ? D / 2 : D;
  __shared__ __attribute__((aligned(16))) float smem[Lay::SMEM];
  // output row of packed row r of head slot hh of the block, at r * hpb + hh
  __shared__ int64_t rowtab[RP * kMaxHeadsPerBlock];

  Work wk0;
  if (!work_of<CAUSAL>(a, wk0)) return;
  const int b = wk0.b, s = wk0.s, hg = wk0.hg, rb = wk0.rg;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int hw = w & (a.hpb - 1);   // this wave's head slot in the group
  const int wk = w >> a.lhpb;       // its index among the waves of that head
  const int wph = NW >> a.lhpb;     // waves per head
  const int g = hg * a.hpb + hw;
  const int r0 = rb * RP;

  Ctx<D, RP> c;
  c.kb = s * a.chunk;
  c.jq = lane / LPK;
  c.qq = lane % LPK;
  c.kg = lane / LPV;
  c.ds = lane % LPV;

  // ---- q rows of this wave's head, in registers (QK layout: chunks qq +
  // LPK*c4), and the split's first page-table window (key windows whose pages
  // fit the LDS page-table slice: one unless the split spans more than kBtCap
  // pages): issued before the sequence's length is used (see work_of)
  QRows<D, RP> qrows;
  {
    const SeqRows &sr0 = wk0.sr;
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      const int rr = r0 + r;
      if (rr < sr0.R) {
        const uint4 *src = reinterpret_cast<const uint4 *>(a.q + out_row(a, sr0.tok0, g, rr) * DO);
        if constexpr (PAIR) {  // the row's D/2 columns in its half (chunks h * D/16 ..), zeros in the other
          const int h = pair_half(a, rr);
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4) {
            const int ch = c.qq + LPK * c4;
            qrows.v[r][c4] = ch / (D / 16) == h ? src[ch % (D / 16)] : make_uint4(0u, 0u, 0u, 0u);
          }
        } else {
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4) qrows.v[r][c4] = src[c.qq + LPK * c4];
        }
      } else {
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) qrows.v[r][c4] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }
  float *pbuf = smem + kBtCap + 4 + w * (T * RP);
  float *kbuf = smem + kBtCap + 4 + Lay::PBUF + w * (T * D / 2);
  int *bt_lds = reinterpret_cast<int *>(smem);
  const int *bt_row = a.block_table + (int64_t)b * a.max_pages;
  const int win_keys = window_keys(kBtCap, a.page_shift, NW * T);
  const int cap_keys = a.max_pages << a.page_shift;
  auto load_bt = [&](int from) {
    if (a.contig) {  // contiguous K/V: sequence b is page b
      if (threadIdx.x == 0) bt_lds[0] = b;
      return;
    }
    int to = from + win_keys;
    if (to > c.kb + a.chunk) to = c.kb + a.chunk;
    if (to > cap_keys) to = cap_keys;
    const int p0 = from >> a.page_shift;
    const int np = to > from ? ((to - 1) >> a.page_shift) - p0 + 1 : 0;
    for (int i = threadIdx.x; i < np; i += NW * 64) bt_lds[i] = bt_row[p0 + i];
  };
  load_bt(c.kb);

  const int L = wk0.L;
  const SeqRows sr = wk0.sr;
  if (r0 >= sr.R) return;  // a row block past the sequence's tokens (varlen batches)

  // per-row visible key limit and the block's key range
  int lim[RP];
  int kmax = 0;
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    lim[r] = row_keys(a, sr, L, r0 + r);
    kmax = lim[r] > kmax ? lim[r] : kmax;
  }

  // splits past the unit's keys: no work; outside the in-kernel merge they
  // leave (m, l) = (-inf, 0) for the combine step
  const int nact = active_splits(a, kmax);
  const int nrows = (sr.R - r0 < RP ? sr.R - r0 : RP) * a.hpb;
  if (s >= nact) {
    if (!a.fused) empty_partials(a, sr.tok0, hg, r0, s, nrows);
    return;
  }
  // the unit's only split with keys writes the output itself
  const bool direct = !a.partials || (a.fused && nact == 1);

  c.kbase = a.k + g * a.head_stride;
  c.vbase = a.v + g * a.head_stride;
  c.bt = reinterpret_cast<const int *>(smem);
  c.page_shift = a.page_shift;
  c.pmask = (1 << a.page_shift) - 1;
  c.page_stride = a.page_stride;
  c.row_stride = a.row_stride;
  c.R = sr.R;
  int kend = c.kb + a.chunk;
  if (kend > kmax) kend = kmax;

  State<RP> st;
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    st.m[r] = -INFINITY;
    st.l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.acc[r][e] = 0.f;
  }

  if ((int)threadIdx.x < RP * a.hpb) {
    const int rr = r0 + (threadIdx.x >> a.lhpb);
    rowtab[threadIdx.x] = rr < sr.R ? out_row(a, sr.tok0, hg * a.hpb + (threadIdx.x & (a.hpb - 1)), rr) : 0;
  }
  __syncthreads();   // the first page-table window (loaded above) is in LDS
  for (int wb = c.kb; wb < kend; wb += win_keys) {
    const int we = wb + win_keys < kend ? wb + win_keys : kend;
    if (wb != c.kb) {
      __syncthreads();
      load_bt(wb);
      __syncthreads();
    }
    c.p0 = wb >> a.page_shift;
    c.ke = we;
    const int ntiles = (we - wb + T - 1) / T;

    tile_loop<D, RP, CAUSAL, MASK, UPAGE>(a, c, b, r0, wb, wk, wph, ntiles, qrows, lim, pbuf, kbuf, st);
  }

  // ---- wave totals: l over QK key groups, acc over PV key groups
  float l_tot[RP];
#pragma unroll
  for (int r = 0; r < RP; ++r) l_tot[r] = reduce_hi_grouped<Lay::LOG_LPK, OpSum>(st.l[r]);
#pragma unroll
  for (int r = 0; r < RP; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) st.acc[r][e] = reduce_hi<Lay::LOG_LPV, OpSum>(st.acc[r][e]);

  // ---- merge the waves of each head through LDS, then write (output, or
  // this split's partial and, fused, the unit's merge by the block that
  // finishes last).  Row slot u = wk * HR + r * hpb + hw: the row index
  // ri = r * hpb + hw of the block's output rows, once per wave of a head.
  __syncthreads();
  const int HR = RP * a.hpb;
  float *ob = smem;                    // [NW * RP][D]
  float *mlb = smem + NW * RP * D;     // [NW * RP][2]
  if (c.kg == 0) {
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      const int u = wk * HR + r * a.hpb + hw;
      float4 *dst = reinterpret_cast<float4 *>(ob + u * D + c.ds * 8);
      dst[0] = make_float4(st.acc[r][0], st.acc[r][1], st.acc[r][2], st.acc[r][3]);
      dst[1] = make_float4(st.acc[r][4], st.acc[r][5], st.acc[r][6], st.acc[r][7]);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      const int u = wk * HR + r * a.hpb + hw;
      *reinterpret_cast<float2 *>(mlb + u * 2) = make_float2(st.m[r], l_tot[r]);
    }
  }
  __syncthreads();
  auto item = [&](int ri, int d, float &M, float &W, float (&v)[8]) {
    // paired: output column d of the row is column d of its half
    const int dd = PAIR ? d + DO * pair_half(a, r0 + (ri >> a.lhpb)) : d;
    merge_waves<NW, D>(mlb, ob, HR, wph, ri, dd, M, W, v);
  };
  write_rows<DO>(a, s, direct, rowtab, nrows, item, NW * 64);
  if (a.fused && !direct) fused_tail<DO>(a, wk0.unit, nact, rowtab, nrows, smem, NW * 64);
}

// Combine (the standalone pkv_combine entry point): each block merges
// combine_rows(D) consecutive rows (one 4-element group per thread) with the
// same merge code as the split kernels' in-kernel merge.
constexpr int combine_rows(int D) { return 1024 / D; }

template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const CombineArgs a) {
  constexpr int NR = combine_rows(D);
  const int64_t base = (int64_t)blockIdx.x * NR;
  const int64_t left = a.rows - base;
  const int nrows = left < NR ? (int)left : NR;
  merge_rows<D, false>(a.o_part, a.ml_part, a.S, a.S, [&](int r) { return base + r; }, nrows, a.out, a.out_f32,
                       256);
}

// Zero-fill (workspace counters); a kernel, not a memset, so it may sit in a
// captured graph.
__global__ __launch_bounds__(256) void zero_kernel(uint32_t *p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

template <int D, int RP, bool C, bool M, bool U, bool PAIR>
hipError_t launch_t(const DecodeArgs &a, hipStream_t stream) {
  const int64_t grid = split_grid(a);
  hipLaunchKernelGGL((split_decode_valu<D, RP, C, M, U, PAIR>), dim3((unsigned)grid), dim3(kWavesPerBlock * 64), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D, int RP, bool C, bool M, bool PAIR = false>
hipError_t launch_u(const DecodeArgs &a, hipStream_t s) {
  // the page of a whole tile is wave-uniform when a page holds at least a tile
  constexpr int T = Layout<D, RP>::T;
  return a.page_shift >= ilog2c(T) ? launch_t<D, RP, C, M, true, PAIR>(a, s) : launch_t<D, RP, C, M, false, PAIR>(a, s);
}

template <int D, int RP, bool PAIR = false>
hipError_t launch_rp(const DecodeArgs &a, bool causal, bool mask, hipStream_t s) {
  if (causal) return mask ? launch_u<D, RP, true, true, PAIR>(a, s) : launch_u<D, RP, true, false, PAIR>(a, s);
  return mask ? launch_u<D, RP, false, true, PAIR>(a, s) : launch_u<D, RP, false, false, PAIR>(a, s);
}

template <int D>
hipError_t launch_d(const DecodeArgs &a, int rp, bool causal, bool mask, hipStream_t s) {
  if constexpr (D == 256) {   // three or four rows per kv head (use_mfma)
    if (rp == 4) return launch_rp<D, 4>(a, causal, mask, s);
  }
  switch (rp) {
    case 1: return launch_rp<D, 1>(a, causal, mask, s);
    default: return launch_rp<D, 2>(a, causal, mask, s);
  }
}

}  // namespace

int launch_split(const DecodeArgs &a, int head_dim, int rp, bool causal, bool has_mask,
                 hipStream_t stream) {
  switch (head_dim) {
    case 32: return launch_d<32>(a, rp, causal, has_mask, stream);
    case 64:  // head pairing: two rows of 64 columns (one query head of each of two kv heads of 32)
      if (a.pair) return rp == 2 ? launch_rp<64, 2, true>(a, causal, has_mask, stream) : hipErrorInvalidValue;
      return launch_d<64>(a, rp, causal, has_mask, stream);
    case 128: return launch_d<128>(a, rp, causal, has_mask, stream);
    default: return launch_d<256>(a, rp, causal, has_mask, stream);
  }
}

int launch_zero(void *p, int64_t words, hipStream_t stream) {
  if (words <= 0) return hipSuccess;
  int64_t blocks = (words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, static_cast<uint32_t *>(p), words);
  return hipGetLastError();
}

int launch_combine(const CombineArgs &a, int head_dim, hipStream_t stream) {
  const int nr = combine_rows(head_dim);
  const unsigned grid = (unsigned)((a.rows + nr - 1) / nr);
  switch (head_dim) {
    case 32: hipLaunchKernelGGL(combine_kernel<32>, dim3(grid), dim3(256), 0, stream, a); break;
    case 64: hipLaunchKernelGGL(combine_kernel<64>, dim3(grid), dim3(256), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(combine_kernel<128>, dim3(grid), dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL(combine_kernel<256>, dim3(grid), dim3(256), 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace pkv
