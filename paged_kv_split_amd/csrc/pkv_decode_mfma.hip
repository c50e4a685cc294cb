// pkv_decode_mfma.hip -- split-KV paged decode kernel for CDNA4 (gfx950),
// matrix-core path, used when the rows that share a kv head (G query heads x
// q_len tokens) fill a 16-row MFMA tile.
//
// Method as in pkv_decode.hip (AstrAI commit d565d44, "attn_paged_decode.cu"
// commit notes: the MMA split-KV paged decode kernel packs the query heads of
// one kv head into tensor-core tiles and resolves the page table once per key
// tile).  gfx950 mapping:
//  * a workgroup covers one key split of up to 32 rows (two 16-row blocks)
//    of each of hpb kv heads (1, 2 or 4); wave w works on head w % hpb and
//    takes every (NW / hpb)-th 16-key tile; the waves of a head merge their
//    (m, l, O) once at the end through LDS;
//  * K and V tiles are fetched with full-row 128-bit loads into registers
//    (double-buffered, so the next tile's loads fly during this tile's math)
//    and written to a per-wave LDS slice with an XOR chunk swizzle;
//  * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: the K operand is a
//    ds_read_b128 per lane, Q stays in registers; the S^T accumulator leaves
//    each lane one query row and four keys, so the online-softmax max, exp
//    and rescale are in-lane apart from two permlane swaps;
//  * O^T = V^T P^T with v_mfma_f32_16x16x16_bf16: V^T comes straight from
//    the row-major V tile through ds_read_b64_tr_b16 (the gfx950 transposing
//    LDS read), P^T is the S^T register layout itself; P is split into a bf16
//    high part and a bf16 remainder (two MFMAs, both converted with the
//    gfx950 v_cvt_pk_bf16_f32) so the probabilities keep about 16
//    significant bits, and the row sums l use the fp32 values;
//  * exclusion (tail, causal, -inf mask) is a select; scores are in base 2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"
#include "pkv_internal.h"
#include "pkv_mfma_tile.h"

namespace pkv {
namespace {

using namespace dev;
using namespace mt;
// One pipeline step: tile tt (in registers tr) -> LDS; issue the loads of
// tile tnext into tr; compute tile tt from LDS.
template <int D, int NRB, bool CAUSAL, bool MASK, bool UPAGE>
__device__ __forceinline__ void mstep(const DecodeArgs &a, const MCtx &c, int b, int r0, int wb, int tt,
                                      int tnext, MTile<D, NRB, MASK> &tr, const uint4 (&qb)[NRB][D / 32],
                                      const int (&lim)[NRB], uint16_t *kt, uint16_t *vt, int lane,
                                      MState<D, NRB> &st) {
  float *mkt = reinterpret_cast<float *>(vt + MLay<D>::TILE_ELEMS);
  mstore<D, NRB, MASK>(tr, kt, vt, mkt, lane);
  // unconditional (a tile past the end loads the last key again, clamped in
  // mload): the loads in flight are then the same on every path, and the
  // wait before the next tile leaves this prefetch in flight
  mload<D, NRB, MASK, UPAGE>(a, c, b, r0, wb + tnext * KT, lane, tr);
  mcompute<D, NRB, CAUSAL, MASK>(a, c, wb + tt * KT, mkt, qb, lim, kt, vt, lane, st);
}

// Register tiles per wave, as measured on MI355X (B = 16 x 4096 keys and
// B = 4 x 32768 keys, Hkv = 8; the 1B-model decode shape): two at D = 32 (the
// 16-key tiles of 1 KB per K or V: 16 x 4096 keys at 32 and 64 query heads
// 22.3 -> 21.3 us) and at D = 64 without a mask (the 1B-model decode shape
// 10.0 -> 9.3 us; with the sweep's mask two were 3-5% slower); two at D = 128
// with a mask (5% faster there); one elsewhere -- at D = 128 without a mask
// one is 7-9% faster and the B = 256 ragged batch (32 rows) 2% faster, and at
// D = 256 two would spill.  More bytes in flight per CU than that made the
// random-page K/V stream slower, not faster (four tiles: up to 60%).
template <int D, int NRB, bool MASK>
constexpr int mfma_nbuf() { return D == 32 ? 2 : D == 64 ? (MASK ? 1 : 2) : (D == 128 && MASK) ? 2 : 1; }

// The key-tile loop of one wave: tiles t0, t0 + tstep, ... < ntiles.
template <int D, int NRB, bool CAUSAL, bool MASK, bool UPAGE, int NBUF = mfma_nbuf<D, NRB, MASK>()>
__device__ __forceinline__ void mtile_loop(const DecodeArgs &a, const MCtx &c, int b, int r0, int wb, int t0,
                                           int tstep, int ntiles, const uint4 (&qb)[NRB][D / 32],
                                           const int (&lim)[NRB], uint16_t *kt, uint16_t *vt, int lane,
                                           MState<D, NRB> &st) {
  // NBUF register tiles in a ring: tile t sits in buffer (t / tstep) % NBUF; a
  // tile goes to LDS, then the loads of the tile NBUF steps ahead are issued
  // into the freed registers
  if (t0 >= ntiles) return;
  MTile<D, NRB, MASK> tr[NBUF];
  // issue the tiles in order, not interleaved by the scheduler, so that the
  // wait for tile i leaves the loads of tiles i+1.. in flight (with fewer
  // tiles than NBUF the extra loads repeat the last key, clamped in mload)
#pragma unroll
  for (int i = 0; i < NBUF; ++i) {
    mload<D, NRB, MASK, UPAGE>(a, c, b, r0, wb + (t0 + i * tstep) * KT, lane, tr[i]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // whole rounds while every prefetch of the round is a tile of this wave:
  // the loads are unconditional and a round has no exit, so the loads in
  // flight are the same on both paths into the loop header (a conditional
  // load or an exit there makes the compiler wait for all loads)
  if constexpr (D == 256) {
    // whole rounds to the end (a step past the last tile computes a tile
    // whose keys all lie past the window end, at weight 0): the peeled form
    // below spilled registers at D = 256 (16 x 4096 keys, 32 query heads:
    // 91.6 -> 98.3 us)
    for (int t = t0; t < ntiles; t += NBUF * tstep) {
#pragma unroll
      for (int i = 0; i < NBUF; ++i) {
        const int tt = t + i * tstep;
        mstep<D, NRB, CAUSAL, MASK, UPAGE>(a, c, b, r0, wb, tt, tt + NBUF * tstep, tr[i], qb, lim, kt, vt, lane,
                                           st);
      }
    }
    return;
  }
  int t = t0;
  for (; t + (2 * NBUF - 1) * tstep < ntiles; t += NBUF * tstep) {
#pragma unroll
    for (int i = 0; i < NBUF; ++i) {
      const int tt = t + i * tstep;
      mstep<D, NRB, CAUSAL, MASK, UPAGE>(a, c, b, r0, wb, tt, tt + NBUF * tstep, tr[i], qb, lim, kt, vt, lane,
                                         st);
    }
  }
  // the last tiles, after the loop: compute the ones that exist and prefetch
  // only tiles that exist, so no load is left in flight past the last tile
  // (its registers would be waited for before the epilogue could reuse them)
  float *mkt = reinterpret_cast<float *>(vt + MLay<D>::TILE_ELEMS);
#pragma unroll
  for (int i = 0; i < NBUF; ++i) {
    const int tt = t + i * tstep;
    if (tt < ntiles) {   // wave-uniform
      mstore<D, NRB, MASK>(tr[i], kt, vt, mkt, lane);
      if (tt + NBUF * tstep < ntiles) mload<D, NRB, MASK, UPAGE>(a, c, b, r0, wb + (tt + NBUF * tstep) * KT, lane, tr[i]);
      mcompute<D, NRB, CAUSAL, MASK>(a, c, wb + tt * KT, mkt, qb, lim, kt, vt, lane, st);
    }
  }
#pragma unroll
  for (int i = 0; i < NBUF; ++i) {
    const int tt = t + (NBUF + i) * tstep;
    if (tt < ntiles) {
      mstore<D, NRB, MASK>(tr[i], kt, vt, mkt, lane);
      mcompute<D, NRB, CAUSAL, MASK>(a, c, wb + tt * KT, mkt, qb, lim, kt, vt, lane, st);
    }
  }
}

// Two resident workgroups per CU (2 waves per SIMD) where the registers allow:
// not with two row blocks at D = 256, nor at D = 128 with a mask (which spills
// within 256 registers).
template <int D, int NRB, bool MASK>
constexpr int mfma_min_blocks() { return (NRB == 2 && (D >= 256 || (D == 128 && MASK))) ? 1 : 2; }

// PAIR: head pairing (pair_half), two kv heads of D/2 columns per head of the
// launch; q, the output and the partials have DO = D/2 columns.
template <int D, int NRB, bool CAUSAL, bool MASK, bool UPAGE, bool PAIR = false>
__global__ __launch_bounds__(kWavesPerBlock * 64, (mfma_min_blocks<D, NRB, MASK>())) void split_decode_mfma(
    const DecodeArgs a) {
  using L = MLay<D>;
  constexpr int NW = L::NW;
  constexpr int DO = PAIR ? D / 2 : D;
  constexpr int RW = 16 * NRB;
  // the merge of the waves takes both row blocks at once (one LDS hand-over)
  constexpr int SMEM = L::MAIN_BYTES > NRB * L::MERGE_BYTES ? L::MAIN_BYTES : NRB * L::MERGE_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[SMEM];
  // output row of packed row rr of head slot hh of the block, at rr * hpb + hh
  __shared__ int64_t rowtab[RW * kMaxHeadsPerBlock];

  Work wk0;
  if (!work_of<CAUSAL>(a, wk0)) return;
  const int b = wk0.b, s = wk0.s, hg = wk0.hg, rg = wk0.rg;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int hw = w & (a.hpb - 1);   // this wave's head slot in the group
  const int wk = w >> a.lhpb;       // its index among the waves of that head
  const int wph = NW >> a.lhpb;     // waves per head
  const int g = hg * a.hpb + hw;
  const int cc = lane & 15;
  const int q = lane >> 4;
  const int r0 = rg * RW;
  const int kb = s * a.chunk;

  int *bt_lds = reinterpret_cast<int *>(smem_raw);
  uint16_t *kt = reinterpret_cast<uint16_t *>(smem_raw + L::BT_BYTES + w * L::WAVE_LDS);
  uint16_t *vt = kt + L::TILE_ELEMS;

  // q operand (lane supplies Q[row cc+16rb][d 32*stp + 8q .. +8]) and the
  // split's first page-table window, issued before the sequence's length is
  // used (see work_of)
  uint4 qb[NRB][D / 32];
  {
    const SeqRows &sr0 = wk0.sr;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int rr = r0 + cc + 16 * rb;
      if (rr < sr0.R) {
        const uint4 *src = reinterpret_cast<const uint4 *>(a.q + out_row(a, sr0.tok0, g, rr) * DO);
        if constexpr (PAIR) {  // the row's D/2 columns in its half (steps h * D/64 ..), zeros in the other
          const int h = pair_half(a, rr);
#pragma unroll
          for (int stp = 0; stp < D / 32; ++stp)
            qb[rb][stp] = (stp / (D / 64)) == h ? src[4 * (stp % (D / 64)) + q] : make_uint4(0u, 0u, 0u, 0u);
        } else {
#pragma unroll
          for (int stp = 0; stp < D / 32; ++stp) qb[rb][stp] = src[4 * stp + q];
        }
      } else {
#pragma unroll
        for (int stp = 0; stp < D / 32; ++stp) qb[rb][stp] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }
  const int *bt_row = a.block_table + (int64_t)b * a.max_pages;
  const int win_keys = window_keys(kBtCap, a.page_shift, NW * KT);
  const int cap_keys = a.max_pages << a.page_shift;
  auto load_bt = [&](int from) {
    if (a.contig) {  // contiguous K/V: sequence b is page b
      if (threadIdx.x == 0) bt_lds[0] = b;
      return;
    }
    int to = from + win_keys;
    if (to > kb + a.chunk) to = kb + a.chunk;
    if (to > cap_keys) to = cap_keys;
    const int p0 = from >> a.page_shift;
    const int np = to > from ? ((to - 1) >> a.page_shift) - p0 + 1 : 0;
    for (int i = threadIdx.x; i < np; i += NW * 64) bt_lds[i] = bt_row[p0 + i];
  };
  load_bt(kb);

  const int kvlen = wk0.L;
  const SeqRows sr = wk0.sr;
  if (r0 >= sr.R) return;  // a row block past the sequence's tokens (varlen batches)
  int lim[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) lim[rb] = row_keys(a, sr, kvlen, r0 + cc + 16 * rb);
  const int rlast = (r0 + RW < sr.R ? r0 + RW : sr.R) - 1;
  const int kmax = row_keys(a, sr, kvlen, rlast);   // the last row sees the most keys

  // splits past the unit's keys: no work; outside the in-kernel merge they
  // leave (m, l) = (-inf, 0) for the combine step
  const int nact = active_splits(a, kmax);
  const int nrt = (sr.R - r0 < RW ? sr.R - r0 : RW) * a.hpb;  // output rows of the block
  if (s >= nact) {
    if (!a.fused) empty_partials(a, sr.tok0, hg, r0, s, nrt);
    return;
  }
  // the unit's only split with keys writes the output itself
  const bool direct = !a.partials || (a.fused && nact == 1);

  MCtx c;
  c.kbase = a.k + g * a.head_stride;
  c.vbase = a.v + g * a.head_stride;
  c.bt = bt_lds;
  c.page_shift = a.page_shift;
  c.pmask = (1 << a.page_shift) - 1;
  c.page_stride = a.page_stride;
  c.row_stride = a.row_stride;
  c.R = sr.R;
  c.kvis = wave_min_limit<NRB>(lim, r0, sr.R, lane);
  int kend = kb + a.chunk;
  if (kend > kmax) kend = kmax;

  MState<D, NRB> st;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    st.m[rb] = -INFINITY;
    st.l[rb] = 0.f;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) st.o[rb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  if ((int)threadIdx.x < RW * a.hpb) {
    const int rr = r0 + (threadIdx.x >> a.lhpb);
    rowtab[threadIdx.x] = rr < sr.R ? out_row(a, sr.tok0, hg * a.hpb + (threadIdx.x & (a.hpb - 1)), rr) : 0;
  }
  __syncthreads();   // the first page-table window (loaded above) is in LDS
  for (int wb = kb; wb < kend; wb += win_keys) {
    const int we = wb + win_keys < kend ? wb + win_keys : kend;
    if (wb != kb) {
      __syncthreads();
      load_bt(wb);
      __syncthreads();
    }
    c.p0 = wb >> a.page_shift;
    c.ke = we;
    const int ntiles = (we - wb + KT - 1) / KT;
    mtile_loop<D, NRB, CAUSAL, MASK, UPAGE>(a, c, b, r0, wb, wk, wph, ntiles, qb, lim, kt, vt, lane, st);
  }

  // row sums over the four lanes of each row
  float ltot[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) ltot[rb] = xor32<OpSum>(xor16<OpSum>(st.l[rb]));

  // merge the waves of each head, both 16-row blocks in one hand-over through
  // LDS, then write every row of the block in one pass (a second pass would
  // first wait for the first pass's global stores to complete).  Row slot
  // u = wk * HR + cc * hpb + hw of row block rb: the block-local row index
  // ri = (16 rb + cc) * hpb + hw (matching rowtab), once per wave of a head.
  const int HR = 16 * a.hpb;
  constexpr int OBN = NW * 16 * L::OB_STRIDE;            // floats per row block
  float *ob = reinterpret_cast<float *>(smem_raw);       // [NRB][NW * 16][OB_STRIDE]
  float *mlb = ob + NRB * OBN;                           // [NRB][NW * 16][2]
  const int u = wk * HR + 16 * hw + cc;   // a wave's rows consecutive (distinct banks for its lanes)
  // columns swizzled at D = 128 (at D <= 64 a pass reads 16 groups of two or
  // more rows already; at D = 256, at the register limit, the swizzled
  // indices spilled more registers)
  constexpr bool OBSW = D == 128;
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) {
      // lane holds O^T[d = 16nb + 4q + i][row cc]
      float4 *dst = OBSW ? reinterpret_cast<float4 *>(ob + rb * OBN + u * L::OB_STRIDE) + ob_unit<true>(4 * nb + q)
                         : reinterpret_cast<float4 *>(ob + rb * OBN + u * L::OB_STRIDE + 16 * nb + 4 * q);
      dst[0] = make_float4(st.o[rb][nb][0], st.o[rb][nb][1], st.o[rb][nb][2], st.o[rb][nb][3]);
    }
    if (q == 0) *reinterpret_cast<float2 *>(mlb + (rb * NW * 16 + u) * 2) = make_float2(st.m[rb], ltot[rb]);
  }
  __syncthreads();
  auto item = [&](int ri, int d, float &M, float &W, float (&v)[8]) {
    const int rb = NRB == 1 ? 0 : ri / HR;
    const int rl = ri - rb * HR;   // (16 rb + cc) * hpb + hw - rb * HR = cc * hpb + hw
    // paired: output column d of the row is column d of its half
    const int dd = PAIR ? d + DO * pair_half(a, r0 + 16 * rb + (rl >> a.lhpb)) : d;
    merge_waves<NW, L::OB_STRIDE, OBSW>(mlb + rb * NW * 16 * 2, ob + rb * OBN, HR, wph,
                                        16 * (rl & (a.hpb - 1)) + (rl >> a.lhpb), dd, M, W, v);
  };
  write_rows<DO>(a, s, direct, rowtab, nrt, item, NW * 64);
  if (a.fused && !direct)
    fused_tail<DO>(a, wk0.unit, nact, rowtab, nrt, reinterpret_cast<float *>(smem_raw), NW * 64);
}

// ---- prefill-shaped workgroup ----------------------------------------------
// Four waves of 32 rows each (128 packed rows of one kv head) over the same
// keys.  A shared tile of 64 keys is four 16-key subtiles, wave w fetching
// subtile w (the same loads and swizzled LDS layout as above); every wave
// then computes all four subtiles for its own rows.  Shared tiles are
// double-buffered in LDS with one barrier per tile: the next tile's loads
// fly while this one computes, and go to LDS after it.  A wave's rows are
// its own, so it writes them (or its split's partials) from registers with
// no merge between waves.  With a mask, each wave stages its rows' mask
// values of the next tile in its own LDS slice after computing the current
// one (single-buffered: only that wave reads it).
template <int D, bool MASK>
struct PLay {
  static constexpr int NW = kWavesPerBlock;
  static constexpr int SUB = NW;                      // 16-key subtiles per shared tile
  static constexpr int KTC = SUB * KT;                // keys per shared tile
  static constexpr int SUB_ELEMS = KT * D;            // bf16 per K (or V) subtile
  static constexpr int BUF_BYTES = 2 * SUB * SUB_ELEMS * 2;
  static constexpr int MASK_SUB = 2 * 64 * 4;         // floats per subtile: [row block][lane] float4
  static constexpr int MASK_WAVE = MASK ? SUB * MASK_SUB * 4 : 0;
  static constexpr int BT_BYTES = (kBtCap + 4) * 4;
  static constexpr int SMEM_BYTES = BT_BYTES + 2 * BUF_BYTES + NW * MASK_WAVE;
};

// Mask values of a wave's rows for the four subtiles of the shared tile at
// key tb: lane (cc, q) takes keys tb + 16 sub + 4q + i of rows rw + cc + 16 rb
// (keys and rows clamped into range; one load per entry on every path).
template <int NRB>
__device__ __forceinline__ void pmask_load(const DecodeArgs &a, const MCtx &c, int b, int rw, int tb, int lane,
                                           float (&pm)[kWavesPerBlock][NRB][4]) {
  const int q = lane >> 4;
  const int cc = lane & 15;
  const int jlast = c.ke - 1;
#pragma unroll
  for (int sub = 0; sub < kWavesPerBlock; ++sub) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int j = tb + KT * sub + 4 * q + i;
      j = j < jlast ? j : jlast;
      const float *mrow = a.mask + (int64_t)b * a.mask_sb + j;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const int rr = rw + cc + 16 * rb < c.R ? rw + cc + 16 * rb : c.R - 1;
        pm[sub][rb][i] = mrow[(int64_t)(rr / a.G) * a.mask_sq];
      }
    }
  }
}

template <int NRB>
__device__ __forceinline__ void pmask_store(const float (&pm)[kWavesPerBlock][NRB][4], float *mw, int lane) {
#pragma unroll
  for (int sub = 0; sub < kWavesPerBlock; ++sub)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
      reinterpret_cast<float4 *>(mw + sub * 2 * 64 * 4)[rb * 64 + lane] =
          make_float4(pm[sub][rb][0], pm[sub][rb][1], pm[sub][rb][2], pm[sub][rb][3]);
  __builtin_amdgcn_wave_barrier();
}

template <int D, bool CAUSAL, bool MASK, bool UPAGE>
__global__ __launch_bounds__(kWavesPerBlock * 64, (MASK && D == 128) ? 1 : 2) void split_prefill_mfma(
    const DecodeArgs a) {
  using P = PLay<D, MASK>;
  constexpr int NW = P::NW;
  constexpr int NRB = 2;                 // 32 rows per wave
  constexpr int RWG = NW * 16 * NRB;     // rows per workgroup
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[P::SMEM_BYTES];
  __shared__ int64_t rowtab[RWG];

  Work wk0;
  if (!work_of<CAUSAL>(a, wk0)) return;
  const int b = wk0.b, s = wk0.s, g = wk0.hg, rg = wk0.rg;  // one kv head per workgroup: group = head
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int cc = lane & 15;
  const int q = lane >> 4;
  const int kvlen = wk0.L;
  const SeqRows sr = wk0.sr;
  const int r0 = rg * RWG;
  if (r0 >= sr.R) return;  // a row block past the sequence's tokens (varlen batches)
  const int rw = r0 + 32 * w;  // this wave's first row
  int lim[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) lim[rb] = row_keys(a, sr, kvlen, rw + cc + 16 * rb);
  const int rlast = (r0 + RWG < sr.R ? r0 + RWG : sr.R) - 1;
  const int kmax = row_keys(a, sr, kvlen, rlast);
  const int wlast = (rw + 32 < sr.R ? rw + 32 : sr.R) - 1;
  const int wkmax = wlast >= rw ? row_keys(a, sr, kvlen, wlast) : 0;  // keys this wave's rows see

  const int nact = active_splits(a, kmax);
  const int nrt = sr.R - r0 < RWG ? sr.R - r0 : RWG;
  if (s >= nact) {
    if (!a.fused) empty_partials(a, sr.tok0, g, r0, s, nrt);
    return;
  }
  const bool direct = !a.partials || (a.fused && nact == 1);

  int *bt_lds = reinterpret_cast<int *>(smem_raw);
  unsigned char *bufs = smem_raw + P::BT_BYTES;
  auto ktile = [&](int buf, int sub) {
    return reinterpret_cast<uint16_t *>(bufs + buf * P::BUF_BYTES) + sub * P::SUB_ELEMS;
  };
  auto vtile = [&](int buf, int sub) {
    return reinterpret_cast<uint16_t *>(bufs + buf * P::BUF_BYTES) + (P::SUB + sub) * P::SUB_ELEMS;
  };
  float *mw = reinterpret_cast<float *>(bufs + 2 * P::BUF_BYTES + w * P::MASK_WAVE);

  MCtx c;
  c.kbase = a.k + g * a.head_stride;
  c.vbase = a.v + g * a.head_stride;
  c.bt = bt_lds;
  c.page_shift = a.page_shift;
  c.pmask = (1 << a.page_shift) - 1;
  c.page_stride = a.page_stride;
  c.row_stride = a.row_stride;
  c.R = sr.R;
  c.kvis = wave_min_limit<NRB>(lim, rw, sr.R, lane);
  const int kb = s * a.chunk;
  int kend = kb + a.chunk;
  if (kend > kmax) kend = kmax;

  uint4 qb[NRB][D / 32];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int rr = rw + cc + 16 * rb;
    if (rr < sr.R) {
      const uint4 *src = reinterpret_cast<const uint4 *>(a.q + out_row(a, sr.tok0, g, rr) * D);
#pragma unroll
      for (int stp = 0; stp < D / 32; ++stp) qb[rb][stp] = src[4 * stp + q];
    } else {
#pragma unroll
      for (int stp = 0; stp < D / 32; ++stp) qb[rb][stp] = make_uint4(0u, 0u, 0u, 0u);
    }
  }

  const int *bt_row = a.block_table + (int64_t)b * a.max_pages;
  const int win_keys = window_keys(kBtCap, a.page_shift, P::KTC);
  const int cap_keys = a.max_pages << a.page_shift;
  auto load_bt = [&](int from) {
    if (a.contig) {  // contiguous K/V: sequence b is page b
      if (threadIdx.x == 0) bt_lds[0] = b;
      return;
    }
    int to = from + win_keys;
    if (to > kb + a.chunk) to = kb + a.chunk;
    if (to > cap_keys) to = cap_keys;
    const int p0 = from >> a.page_shift;
    const int np = to > from ? ((to - 1) >> a.page_shift) - p0 + 1 : 0;
    for (int i = threadIdx.x; i < np; i += NW * 64) bt_lds[i] = bt_row[p0 + i];
  };

  MState<D, NRB> st;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    st.m[rb] = -INFINITY;
    st.l[rb] = 0.f;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) st.o[rb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  if (threadIdx.x < RWG) {
    const int rr = r0 + threadIdx.x;
    rowtab[threadIdx.x] = rr < sr.R ? out_row(a, sr.tok0, g, rr) : 0;
  }
  load_bt(kb);
  __syncthreads();
  for (int wb = kb; wb < kend; wb += win_keys) {
    const int we = wb + win_keys < kend ? wb + win_keys : kend;
    if (wb != kb) {
      __syncthreads();
      load_bt(wb);
      __syncthreads();
    }
    c.p0 = wb >> a.page_shift;
    c.ke = we;
    const int ntiles = (we - wb + P::KTC - 1) / P::KTC;
    MTile<D, NRB, false> tr;
    float pm[MASK ? NW : 1][NRB][4];
    mload<D, NRB, false, UPAGE, true>(a, c, b, rw, wb + KT * w, lane, tr);
    if constexpr (MASK) pmask_load<NRB>(a, c, b, rw, wb, lane, pm);
    mstore<D, NRB, false>(tr, ktile(0, w), vtile(0, w), nullptr, lane);
    if constexpr (MASK) pmask_store<NRB>(pm, mw, lane);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      const int buf = t & 1;
      const int tb = wb + t * P::KTC;
      // the next shared tile (unconditional: past the window end, mload and
      // pmask_load clamp to its last key)
      mload<D, NRB, false, UPAGE, true>(a, c, b, rw, tb + P::KTC + KT * w, lane, tr);
      if constexpr (MASK) pmask_load<NRB>(a, c, b, rw, tb + P::KTC, lane, pm);
#pragma unroll
      for (int sub = 0; sub < P::SUB; sub += 2) {
        const int base = tb + KT * sub;
        if (base < wkmax)  // wave-uniform: some row of this wave sees a key of the subtile pair
          mcompute2<D, NRB, CAUSAL, MASK, true>(a, c, base, mw + sub * P::MASK_SUB, mw + (sub + 1) * P::MASK_SUB,
                                                qb, lim, ktile(buf, sub), vtile(buf, sub), ktile(buf, sub + 1),
                                                vtile(buf, sub + 1), lane, st);
      }
      mstore<D, NRB, false>(tr, ktile(buf ^ 1, w), vtile(buf ^ 1, w), nullptr, lane);
      if constexpr (MASK) pmask_store<NRB>(pm, mw, lane);
      __syncthreads();
    }
  }

  // each wave writes its own rows: lane (cc, q) holds O^T[16nb + 4q + i][row cc]
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const float W = xor32<OpSum>(xor16<OpSum>(st.l[rb]));
    const int rr = rw + 16 * rb + cc;
    if (rr < sr.R) {
      const int64_t row = out_row(a, sr.tok0, g, rr);
      const float inv = W > 0.f ? 1.f / W : 0.f;
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) {
        const int d0 = 16 * nb + 4 * q;
        const f32x4_t v = st.o[rb][nb] * inv;
        if (direct) {
          const uint32_t lo = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
          const uint32_t hi = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
          *reinterpret_cast<uint2 *>(a.out + row * D + d0) = make_uint2(lo, hi);
          if (a.out_f32) *reinterpret_cast<float4 *>(a.out_f32 + row * D + d0) = make_float4(v[0], v[1], v[2], v[3]);
        } else if (W > 0.f) {
          float *po = a.o_part + (row * a.S + s) * D + d0;
          if (a.fused) {  // merged by another workgroup of this launch
            store_part4(a, po, v[0], v[1], v[2], v[3]);
          } else {
            *reinterpret_cast<float4 *>(po) = make_float4(v[0], v[1], v[2], v[3]);
          }
        }
      }
      if (!direct && q == 0) {
        float *pm2 = a.ml_part + (row * a.S + s) * 2;
        const float mx = W > 0.f ? st.m[rb] * kLn2 : -INFINITY;
        if (a.fused)
          store_dev2(pm2, mx, W);
        else
          *reinterpret_cast<float2 *>(pm2) = make_float2(mx, W);
      }
    }
  }
  if (a.fused && !direct)
    fused_tail<D>(a, wk0.unit, nact, rowtab, nrt, reinterpret_cast<float *>(smem_raw), NW * 64);
}

template <int D, bool C, bool M, bool U>
hipError_t plaunch_t(const DecodeArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL((split_prefill_mfma<D, C, M, U>), dim3((unsigned)split_grid(a)), dim3(kWavesPerBlock * 64), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D, bool C, bool M>
hipError_t plaunch_u(const DecodeArgs &a, hipStream_t s) {
  return a.page_shift >= 4 ? plaunch_t<D, C, M, true>(a, s) : plaunch_t<D, C, M, false>(a, s);
}

template <int D>
hipError_t plaunch_d(const DecodeArgs &a, bool causal, bool mask, hipStream_t s) {
  if (causal) return mask ? plaunch_u<D, true, true>(a, s) : plaunch_u<D, true, false>(a, s);
  return mask ? plaunch_u<D, false, true>(a, s) : plaunch_u<D, false, false>(a, s);
}

template <int D, int NRB, bool C, bool M, bool U, bool PAIR>
hipError_t mlaunch_t(const DecodeArgs &a, hipStream_t stream) {
  const int64_t grid = split_grid(a);
  hipLaunchKernelGGL((split_decode_mfma<D, NRB, C, M, U, PAIR>), dim3((unsigned)grid), dim3(kWavesPerBlock * 64),
                     0, stream, a);
  return hipGetLastError();
}

template <int D, int NRB, bool C, bool M, bool PAIR = false>
hipError_t mlaunch_u(const DecodeArgs &a, hipStream_t s) {
  // a 16-key tile's page is wave-uniform when pages hold at least 16 keys
  return a.page_shift >= 4 ? mlaunch_t<D, NRB, C, M, true, PAIR>(a, s) : mlaunch_t<D, NRB, C, M, false, PAIR>(a, s);
}

template <int D, int NRB, bool PAIR = false>
hipError_t mlaunch_nrb(const DecodeArgs &a, bool causal, bool mask, hipStream_t s) {
  if (causal) return mask ? mlaunch_u<D, NRB, true, true, PAIR>(a, s) : mlaunch_u<D, NRB, true, false, PAIR>(a, s);
  return mask ? mlaunch_u<D, NRB, false, true, PAIR>(a, s) : mlaunch_u<D, NRB, false, false, PAIR>(a, s);
}

template <int D>
hipError_t mlaunch_d(const DecodeArgs &a, int nrb16, bool causal, bool mask, hipStream_t s) {
  return nrb16 == 1 ? mlaunch_nrb<D, 1>(a, causal, mask, s) : mlaunch_nrb<D, 2>(a, causal, mask, s);
}

}  // namespace

int launch_split_prefill(const DecodeArgs &a, int head_dim, bool causal, bool has_mask, hipStream_t stream) {
  switch (head_dim) {
    case 32: return plaunch_d<32>(a, causal, has_mask, stream);
    case 64: return plaunch_d<64>(a, causal, has_mask, stream);
    default: return plaunch_d<128>(a, causal, has_mask, stream);
  }
}

int launch_split_mfma(const DecodeArgs &a, int head_dim, int nrb16, bool causal, bool has_mask,
                      hipStream_t stream) {
  switch (head_dim) {
    case 32: return mlaunch_d<32>(a, nrb16, causal, has_mask, stream);
    case 64:  // head pairing: one 16-row block of 64 columns (two kv heads of 32)
      if (a.pair) return nrb16 == 1 ? mlaunch_nrb<64, 1, true>(a, causal, has_mask, stream) : hipErrorInvalidValue;
      return mlaunch_d<64>(a, nrb16, causal, has_mask, stream);
    case 128: return mlaunch_d<128>(a, nrb16, causal, has_mask, stream);
    default: return mlaunch_d<256>(a, nrb16, causal, has_mask, stream);
  }
}

}  // namespace pkv
