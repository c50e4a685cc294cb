// pkv_decode_group.hip -- split-KV paged decode kernel for CDNA4 (gfx950),
// matrix-core path with K/V tiles shared by the workgroup across a group of
// kv heads.
//
// Method as in pkv_decode.hip (AstrAI commit d565d44, "attn_paged_decode.cu"
// commit notes: the MMA split-KV paged decode kernel packs the query heads of
// one kv head into tensor-core tiles, stages K and V in shared memory and
// double-buffers them so the next tile's loads overlap this tile's math).
// gfx950 mapping:
//  * a workgroup covers one key split of HG = 4 * HW consecutive kv heads
//    (4 or 8) and up to 16 * NRB packed rows of each; its four waves each own
//    HW of the heads, all rows and all keys of the split, so no merge between
//    waves is needed;
//  * a shared tile is TK keys of the whole head group: for each key, the
//    group's HG * D elements are one contiguous run of the page slot (a whole
//    slot when HG = Hkv), and consecutive keys of a page are neighbours, so
//    the workgroup reads runs of HG * D * 2 bytes per key -- 256 B to 1 KB
//    and more across the keys of a page -- where a one-head workgroup reads
//    separate 64 to 256-byte head slices, which HBM serves more slowly;
//  * the 256 threads load the next two tiles into registers (up to four
//    128-bit loads of K and four of V each per tile, whole rows, 1 KB per wave
//    instruction) while the waves compute the current one from LDS; then the
//    next tile's registers go to the other LDS buffer as per-head 16-key
//    subtiles in the swizzled layout of the one-head kernel, and one barrier
//    per tile hands them over;
//  * each wave computes its heads' subtiles with the matrix-core tile code
//    shared with the one-head kernel (pkv_mfma_tile.h), pairs of subtiles as
//    one 16x16x32 PV product per 16 columns;
//  * mask values (per row and key) go through each wave's own LDS slice, one
//    tile ahead, as in the prefill-shaped kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"
#include "pkv_internal.h"
#include "pkv_mfma_tile.h"

namespace pkv {
namespace {

using namespace dev;
using namespace mt;

// LDS bytes of a workgroup: page-table window, two tile buffers (K and V of
// `subs` 16-key subtiles of HG heads), and each wave's mask slice.
constexpr int group_smem(int D, int HG, int NRB, bool MASK, int subs) {
  return (kBtCap + 4) * 4 + 2 * (2 * subs * HG * KT * D * 2) + (MASK ? kWavesPerBlock * subs * NRB * 64 * 16 : 0);
}

// 16-key subtiles per shared tile: 8192 elements of K per tile (32 KB of K
// and V per buffer; a whole tile is then four 128-bit loads of K and four of
// V per thread), at most 4 subtiles, halved while the workgroup would take
// more than 80 KB of LDS (two workgroups per CU).
constexpr int group_subs(int D, int HG, int NRB, bool MASK) {
  int s = 8192 / (HG * D * KT);
  s = s < 1 ? 1 : (s > 4 ? 4 : s);
  while (s > 1 && group_smem(D, HG, NRB, MASK, s) > 80 * 1024) s /= 2;
  return s;
}

template <int D, int HW, int NRB, bool MASK>
struct GLay {
  static constexpr int NW = kWavesPerBlock;
  static constexpr int HG = NW * HW;                 // kv heads per workgroup
  static constexpr int CPR = HG * D / 8;             // 16-byte chunks of a key's group row
  static constexpr int SUBS = group_subs(D, HG, NRB, MASK);  // 16-key subtiles per tile
  static constexpr int TK = SUBS * KT;               // keys per shared tile
  static constexpr int NL = TK * CPR / (NW * 64);    // 128-bit loads per thread per tile (K; as many V)
  static constexpr int SUB_ELEMS = KT * D;           // bf16 per head subtile
  static constexpr int HALF_ELEMS = SUBS * HG * SUB_ELEMS;   // K (or V) of one buffer
  static constexpr int BUF_BYTES = 2 * HALF_ELEMS * 2;
  static constexpr int MASK_SUB = NRB * 64 * 4;      // floats per subtile and wave: [row block][lane] float4
  static constexpr int MASK_WAVE = MASK ? SUBS * MASK_SUB * 4 : 0;   // bytes
  static constexpr int BT_BYTES = (kBtCap + 4) * 4;
  static constexpr int SMEM_BYTES = BT_BYTES + 2 * BUF_BYTES + NW * MASK_WAVE;
  static_assert(SMEM_BYTES == group_smem(D, HG, NRB, MASK, SUBS), "LDS layout");
  static_assert(NL * NW * 64 == TK * CPR, "the loads of a tile cover it once");
  static_assert(CPR <= NW * 64, "a key's group row fits one pass of the workgroup");
};

// Where this thread's 16-byte pieces of a tile sit: piece i is chunk
// f = i * 256 + tid of the tile, the chunk f % CPR of key f / CPR; its
// element offset from the group's first head (head stride, then the chunk
// within the head's row) is the same for every tile.
template <int D, int HW, int NRB, bool MASK>
struct GMap {
  using L = GLay<D, HW, NRB, MASK>;
  int key[L::NL];       // key within the tile
  int64_t hofs[L::NL];  // element offset of the chunk from the group's first head at that key
  __device__ void init(const DecodeArgs &a) {
#pragma unroll
    for (int i = 0; i < L::NL; ++i) {
      const int f = i * L::NW * 64 + (int)threadIdx.x;
      const int c = f % L::CPR;
      key[i] = f / L::CPR;
      hofs[i] = (int64_t)(c / (D / 8)) * a.head_stride + 8 * (c % (D / 8));
    }
  }
};

template <int D, int HW, int NRB, bool MASK>
struct GTile {
  uint4 k[GLay<D, HW, NRB, MASK>::NL];
  uint4 v[GLay<D, HW, NRB, MASK>::NL];
};

// Loads of the shared tile at key base: keys past the window end are clamped
// to its last key (finite data, zero weight).  With UPAGE (a page holds a
// whole tile, and tiles start on tile boundaries) the tile's page is resolved
// once, in scalar registers.
template <int D, int HW, int NRB, bool MASK, bool UPAGE>
__device__ __forceinline__ void gload(const MCtx &c, const GMap<D, HW, NRB, MASK> &mp, int base,
                                      GTile<D, HW, NRB, MASK> &t) {
  using L = GLay<D, HW, NRB, MASK>;
  const int jlast = c.ke - 1;
  if constexpr (UPAGE) {
    const int bj = base < jlast ? base : jlast;
    const int page = __builtin_amdgcn_readfirstlane(c.bt[(bj >> c.page_shift) - c.p0]);
    const int64_t pofs = (int64_t)page * c.page_stride + (int64_t)(bj & c.pmask) * c.row_stride;
    const uint16_t *kp = c.kbase + pofs;
    const uint16_t *vp = c.vbase + pofs;
#pragma unroll
    for (int i = 0; i < L::NL; ++i) {
      int j = base + mp.key[i];
      j = j < jlast ? j : jlast;
      const int64_t off = (int64_t)(j - bj) * c.row_stride + mp.hofs[i];
      t.k[i] = load_stream(reinterpret_cast<const uint4 *>(kp + off));
      t.v[i] = load_stream(reinterpret_cast<const uint4 *>(vp + off));
    }
  } else {
#pragma unroll
    for (int i = 0; i < L::NL; ++i) {
      int j = base + mp.key[i];
      j = j < jlast ? j : jlast;
      const int page = c.bt[(j >> c.page_shift) - c.p0];
      const int64_t off = (int64_t)page * c.page_stride + (int64_t)(j & c.pmask) * c.row_stride + mp.hofs[i];
      t.k[i] = load_stream(reinterpret_cast<const uint4 *>(c.kbase + off));
      t.v[i] = load_stream(reinterpret_cast<const uint4 *>(c.vbase + off));
    }
  }
}

// Registers of a tile -> LDS buffer `buf` as per-head 16-key subtiles
// [sub][head][16 rows][D] (K, then V), rows swizzled as in the one-head kernel.
template <int D, int HW, int NRB, bool MASK>
__device__ __forceinline__ void gstore(const GTile<D, HW, NRB, MASK> &t, uint16_t *buf) {
  using L = GLay<D, HW, NRB, MASK>;
  using M = MLay<D>;
#pragma unroll
  for (int i = 0; i < L::NL; ++i) {
    const int f = i * L::NW * 64 + (int)threadIdx.x;
    const int key = f / L::CPR;
    const int c = f % L::CPR;
    const int head = c / (D / 8);
    const int ch = c % (D / 8);
    const int row = key % KT;
    uint16_t *kt = buf + (((key / KT) * L::HG + head) * KT + row) * D;
    reinterpret_cast<uint4 *>(kt)[M::swk(ch, row)] = t.k[i];
    reinterpret_cast<uint4 *>(kt + L::HALF_ELEMS)[M::swv(ch, row)] = t.v[i];
  }
}

// Mask values of a wave's rows for the SUBS subtiles of the tile at key tb:
// lane (cc, q) takes keys tb + 16 sub + 4q + i of rows r0 + cc + 16 rb (keys
// and rows clamped into range; one load per entry on every path).
template <int SUBS, int NRB>
__device__ __forceinline__ void gmask_load(const DecodeArgs &a, const MCtx &c, int b, int r0, int tb, int lane,
                                           float (&pm)[SUBS][NRB][4]) {
  const int q = lane >> 4;
  const int cc = lane & 15;
  const int jlast = c.ke - 1;
#pragma unroll
  for (int sub = 0; sub < SUBS; ++sub) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int j = tb + KT * sub + 4 * q + i;
      j = j < jlast ? j : jlast;
      const float *mrow = a.mask + (int64_t)b * a.mask_sb + j;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const int rr = r0 + cc + 16 * rb < c.R ? r0 + cc + 16 * rb : c.R - 1;
        pm[sub][rb][i] = mrow[(int64_t)(rr / a.G) * a.mask_sq];
      }
    }
  }
}

template <int SUBS, int NRB>
__device__ __forceinline__ void gmask_store(const float (&pm)[SUBS][NRB][4], float *mw, int lane) {
#pragma unroll
  for (int sub = 0; sub < SUBS; ++sub)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
      reinterpret_cast<float4 *>(mw + sub * NRB * 64 * 4)[rb * 64 + lane] =
          make_float4(pm[sub][rb][0], pm[sub][rb][1], pm[sub][rb][2], pm[sub][rb][3]);
  __builtin_amdgcn_wave_barrier();
}

template <int D, int HW, int NRB, bool CAUSAL, bool MASK, bool UPAGE>
__global__ __launch_bounds__(kWavesPerBlock * 64, 2) void split_decode_group(const DecodeArgs a) {
  using L = GLay<D, HW, NRB, MASK>;
  constexpr int NW = L::NW;
  constexpr int HG = L::HG;
  constexpr int RW = 16 * NRB;          // packed rows per head
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[L::SMEM_BYTES];
  // output row of packed row r of head slot hh of the block, at r * HG + hh
  __shared__ int64_t rowtab[RW * HG];

  Work wk0;
  if (!work_of<CAUSAL>(a, wk0)) return;
  const int b = wk0.b, s = wk0.s, hg = wk0.hg, rg = wk0.rg;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int cc = lane & 15;
  const int q = lane >> 4;
  const int r0 = rg * RW;
  const int kvlen = wk0.L;
  const SeqRows sr = wk0.sr;
  if (r0 >= sr.R) return;  // a row block past the sequence's tokens (varlen batches)
  int lim[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) lim[rb] = row_keys(a, sr, kvlen, r0 + cc + 16 * rb);
  const int rlast = (r0 + RW < sr.R ? r0 + RW : sr.R) - 1;
  const int kmax = row_keys(a, sr, kvlen, rlast);   // the last row sees the most keys

  const int nact = active_splits(a, kmax);
  const int nr = sr.R - r0 < RW ? sr.R - r0 : RW;   // rows per head in this block
  const int nrt = nr * HG;                          // output rows of the block
  if (s >= nact) {
    if (!a.fused) empty_partials(a, sr.tok0, hg, r0, s, nrt);
    return;
  }
  const bool direct = !a.partials || (a.fused && nact == 1);

  int *bt_lds = reinterpret_cast<int *>(smem_raw);
  uint16_t *bufs = reinterpret_cast<uint16_t *>(smem_raw + L::BT_BYTES);
  float *mw = reinterpret_cast<float *>(smem_raw + L::BT_BYTES + 2 * L::BUF_BYTES + w * L::MASK_WAVE);
  auto kt = [&](int buf, int sub, int head) {
    return bufs + buf * (L::BUF_BYTES / 2) + (sub * HG + head) * L::SUB_ELEMS;
  };
  auto vt = [&](int buf, int sub, int head) { return kt(buf, sub, head) + L::HALF_ELEMS; };

  MCtx c;
  c.kbase = a.k + (int64_t)hg * HG * a.head_stride;
  c.vbase = a.v + (int64_t)hg * HG * a.head_stride;
  c.bt = bt_lds;
  c.page_shift = a.page_shift;
  c.pmask = (1 << a.page_shift) - 1;
  c.page_stride = a.page_stride;
  c.row_stride = a.row_stride;
  c.R = sr.R;
  c.kvis = wave_min_limit<NRB>(lim, r0, sr.R, lane);
  const int kb = s * a.chunk;
  int kend = kb + a.chunk;
  if (kend > kmax) kend = kmax;

  GMap<D, HW, NRB, MASK> mp;
  mp.init(a);

  // q operands of this wave's heads: lane supplies Q[row cc+16rb][d 32*stp + 8q .. +8]
  uint4 qb[HW][NRB][D / 32];
#pragma unroll
  for (int j = 0; j < HW; ++j) {
    const int g = hg * HG + w * HW + j;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int rr = r0 + cc + 16 * rb;
      if (rr < sr.R) {
        const uint4 *src = reinterpret_cast<const uint4 *>(a.q + out_row(a, sr.tok0, g, rr) * D);
#pragma unroll
        for (int stp = 0; stp < D / 32; ++stp) qb[j][rb][stp] = src[4 * stp + q];
      } else {
#pragma unroll
        for (int stp = 0; stp < D / 32; ++stp) qb[j][rb][stp] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }

  const int *bt_row = a.block_table + (int64_t)b * a.max_pages;
  const int win_keys = window_keys(kBtCap, a.page_shift, L::TK);
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

  MState<D, NRB> st[HW];
#pragma unroll
  for (int j = 0; j < HW; ++j)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      st[j].m[rb] = -INFINITY;
      st[j].l[rb] = 0.f;
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) st[j].o[rb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  if ((int)threadIdx.x < RW * HG) {
    const int rr = r0 + (int)threadIdx.x / HG;
    rowtab[threadIdx.x] = rr < sr.R ? out_row(a, sr.tok0, hg * HG + (int)threadIdx.x % HG, rr) : 0;
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
    const int ntiles = (we - wb + L::TK - 1) / L::TK;
    // Two register tiles in a ring ahead of the two LDS buffers: while tile
    // tt computes from LDS, the loads of tiles tt + 1 and tt + 2 are in
    // flight.  After computing tt, the workgroup stores tile tt + 1 into the
    // other LDS buffer (last read while computing tt - 1, before the previous
    // barrier), passes one barrier, and issues the loads of tile tt + 3 into
    // the registers it freed.  Loads are unconditional and the loop runs whole
    // pairs of tiles (a tile past the window end loads its last key again and
    // its computation is skipped), so the loads in flight are the same on
    // every path.
    GTile<D, HW, NRB, MASK> tr0, tr1;
    float pm0[MASK ? L::SUBS : 1][NRB][4], pm1[MASK ? L::SUBS : 1][NRB][4];
    gload<D, HW, NRB, MASK, UPAGE>(c, mp, wb, tr0);
    if constexpr (MASK) gmask_load<L::SUBS, NRB>(a, c, b, r0, wb, lane, pm0);
    __builtin_amdgcn_sched_barrier(0);
    gload<D, HW, NRB, MASK, UPAGE>(c, mp, wb + L::TK, tr1);
    if constexpr (MASK) gmask_load<L::SUBS, NRB>(a, c, b, r0, wb + L::TK, lane, pm1);
    __builtin_amdgcn_sched_barrier(0);
    gstore<D, HW, NRB, MASK>(tr0, bufs);
    if constexpr (MASK) gmask_store<L::SUBS, NRB>(pm0, mw, lane);
    __syncthreads();
    gload<D, HW, NRB, MASK, UPAGE>(c, mp, wb + 2 * L::TK, tr0);
    if constexpr (MASK) gmask_load<L::SUBS, NRB>(a, c, b, r0, wb + 2 * L::TK, lane, pm0);
    __builtin_amdgcn_sched_barrier(0);
    // one step: compute tile tt from LDS buffer `buf`; tile tt + 1 (in `nx`)
    // to the other buffer; barrier; the loads of tile tt + 3 into `nx`
    auto step = [&](int tt, int buf, GTile<D, HW, NRB, MASK> &nx, float (&pmn)[MASK ? L::SUBS : 1][NRB][4]) {
      const int tb = wb + tt * L::TK;
      if constexpr (L::SUBS >= 2) {
#pragma unroll
        for (int sub = 0; sub < L::SUBS; sub += 2) {
          const int base = tb + KT * sub;
          if (base < we) {  // wave-uniform: the pair holds keys of the window
#pragma unroll
            for (int j = 0; j < HW; ++j)
              mcompute2<D, NRB, CAUSAL, MASK>(a, c, base, mw + sub * L::MASK_SUB, mw + (sub + 1) * L::MASK_SUB,
                                              qb[j], lim, kt(buf, sub, w * HW + j), vt(buf, sub, w * HW + j),
                                              kt(buf, sub + 1, w * HW + j), vt(buf, sub + 1, w * HW + j), lane,
                                              st[j]);
          }
        }
      } else {
        if (tb < we) {
#pragma unroll
          for (int j = 0; j < HW; ++j)
            mcompute<D, NRB, CAUSAL, MASK>(a, c, tb, mw, qb[j], lim, kt(buf, 0, w * HW + j),
                                           vt(buf, 0, w * HW + j), lane, st[j]);
        }
      }
      gstore<D, HW, NRB, MASK>(nx, bufs + (buf ^ 1) * (L::BUF_BYTES / 2));
      if constexpr (MASK) gmask_store<L::SUBS, NRB>(pmn, mw, lane);
      __syncthreads();
      gload<D, HW, NRB, MASK, UPAGE>(c, mp, tb + 3 * L::TK, nx);
      if constexpr (MASK) gmask_load<L::SUBS, NRB>(a, c, b, r0, tb + 3 * L::TK, lane, pmn);
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int t = 0; t < ntiles; t += 2) {
      step(t, 0, tr1, pm1);
      step(t + 1, 1, tr0, pm0);
    }
  }

  // each wave writes its heads' rows: lane (cc, q) holds O^T[16nb + 4q + i][row cc]
#pragma unroll
  for (int j = 0; j < HW; ++j) {
    const int g = hg * HG + w * HW + j;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const float W = xor32<OpSum>(xor16<OpSum>(st[j].l[rb]));
      const int rr = r0 + 16 * rb + cc;
      if (rr < sr.R) {
        const int64_t row = out_row(a, sr.tok0, g, rr);
        const float inv = W > 0.f ? 1.f / W : 0.f;
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) {
          const int d0 = 16 * nb + 4 * q;
          const f32x4_t v = st[j].o[rb][nb] * inv;
          if (direct) {
            const uint32_t lo = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
            const uint32_t hi = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
            *reinterpret_cast<uint2 *>(a.out + row * D + d0) = make_uint2(lo, hi);
            if (a.out_f32)
              *reinterpret_cast<float4 *>(a.out_f32 + row * D + d0) = make_float4(v[0], v[1], v[2], v[3]);
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
          const float mx = W > 0.f ? st[j].m[rb] * kLn2 : -INFINITY;
          if (a.fused)
            store_dev2(pm2, mx, W);
          else
            *reinterpret_cast<float2 *>(pm2) = make_float2(mx, W);
        }
      }
    }
  }
  if (a.fused && !direct)
    fused_tail<D>(a, wk0.unit, nact, rowtab, nrt, reinterpret_cast<float *>(smem_raw), NW * 64);
}

template <int D, int HW, int NRB, bool C, bool M, bool U>
hipError_t glaunch_t(const DecodeArgs &a, hipStream_t stream) {
  hipLaunchKernelGGL((split_decode_group<D, HW, NRB, C, M, U>), dim3((unsigned)split_grid(a)),
                     dim3(kWavesPerBlock * 64), 0, stream, a);
  return hipGetLastError();
}

template <int D, int HW, int NRB, bool C, bool M>
hipError_t glaunch_u(const DecodeArgs &a, hipStream_t s) {
  // a tile's page is wave-uniform when pages hold at least a tile
  constexpr int TK = GLay<D, HW, NRB, M>::TK;
  constexpr int LTK = TK == 16 ? 4 : TK == 32 ? 5 : 6;
  return a.page_shift >= LTK ? glaunch_t<D, HW, NRB, C, M, true>(a, s) : glaunch_t<D, HW, NRB, C, M, false>(a, s);
}

template <int D, int HW, int NRB>
hipError_t glaunch_nrb(const DecodeArgs &a, bool causal, bool mask, hipStream_t s) {
  if (causal) return mask ? glaunch_u<D, HW, NRB, true, true>(a, s) : glaunch_u<D, HW, NRB, true, false>(a, s);
  return mask ? glaunch_u<D, HW, NRB, false, true>(a, s) : glaunch_u<D, HW, NRB, false, false>(a, s);
}

template <int D, int HW>
hipError_t glaunch_hw(const DecodeArgs &a, int nrb16, bool causal, bool mask, hipStream_t s) {
  return nrb16 == 1 ? glaunch_nrb<D, HW, 1>(a, causal, mask, s) : glaunch_nrb<D, HW, 2>(a, causal, mask, s);
}

}  // namespace

int launch_split_group(const DecodeArgs &a, int head_dim, int nrb16, bool causal, bool has_mask,
                       hipStream_t stream) {
  const bool eight = a.hpb == 8;
  switch (head_dim) {
    case 32:
      return eight ? glaunch_hw<32, 2>(a, nrb16, causal, has_mask, stream)
                   : glaunch_hw<32, 1>(a, nrb16, causal, has_mask, stream);
    case 64:
      return eight ? glaunch_hw<64, 2>(a, nrb16, causal, has_mask, stream)
                   : glaunch_hw<64, 1>(a, nrb16, causal, has_mask, stream);
    default:
      return glaunch_hw<128, 1>(a, nrb16, causal, has_mask, stream);
  }
}

}  // namespace pkv
