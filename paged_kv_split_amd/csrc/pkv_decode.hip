// pkv_decode.hip -- split-KV paged decode kernel for CDNA4 (gfx950), VALU path.
//
// Method (AstrAI commit d565d44, "csrc/kernels/attn_paged_decode.cu", commit
// notes on the scalar split-KV paged decode kernel and the MMA variant): every
// workgroup takes one (sequence b, kv head g, key split s, row block) unit.
// The query rows that share kv head g (G query heads x q_len tokens: "GQA head
// packing") are processed together, so every K/V byte is read from HBM once
// per unit.  Keys are resolved through the page table, scores are accumulated
// with an online softmax (running max m and sum l per row), and the split
// leaves either the final output (one split) or a normalised partial plus
// (m, l) for the combine kernel.
//
// gfx950 mapping:
//  * a workgroup is kWavesPerBlock wave64s; wave w takes tiles w, w+NW, ...
//    of T keys and keeps its own (m, l, acc); waves merge once at the end
//    through LDS, so the key loop has no workgroup barrier;
//  * QK^T uses v_dot2_f32_bf16 on packed bf16 pairs (exact products, fp32
//    accumulation) in a "key-major" lane layout: D/32 lanes per key, each
//    holding 32 elements of q and k, reduced across those lanes;
//  * PV uses fp32 FMAs in a "d-major" layout: D/8 lanes per key, each owning
//    8 output columns; probabilities cross between the two layouts through a
//    per-wave LDS slice (no barrier: LDS is in order within a wave);
//  * K and V rows are fetched with 128-bit loads, one page-table lookup per
//    key row, 64-bit element offsets; rows past the split end are never
//    loaded (tails read as zero);
//  * the workgroup index is decoded so that the Hkv x row-block siblings of a
//    (b, s) unit land on the same XCD back to back (blocks are dealt to the 8
//    XCDs round-robin), so they share that XCD's L2 for the interleaved kv
//    heads of a page slot;
//  * scores live in base 2 (scale * log2 e folded in) and use v_exp_f32;
//    exclusion (tail, causal, -inf mask) is a select, never an add.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_internal.h"

namespace pkv {

int rows_per_block(int R) {
  if (R <= 1) return 1;
  if (R <= 2) return 2;
  if (R <= 4) return 4;
  return 8;
}

int tile_keys(int head_dim) { return 2 * (64 / (head_dim / 32)); }

namespace {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}
__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr int ilog2c(int x) { return x <= 1 ? 0 : 1 + ilog2c(x / 2); }

// max / sum over the lanes that differ in lane-id bits [LO, 6)
template <int LO>
__device__ __forceinline__ float wave_max_hi(float x) {
#pragma unroll
  for (int bit = LO; bit < 6; ++bit) x = fmaxf(x, __shfl_xor(x, 1 << bit, 64));
  return x;
}
template <int LO>
__device__ __forceinline__ float wave_sum_hi(float x) {
#pragma unroll
  for (int bit = LO; bit < 6; ++bit) x += __shfl_xor(x, 1 << bit, 64);
  return x;
}
// sum over the lanes that differ in lane-id bits [0, HI)
template <int HI>
__device__ __forceinline__ float wave_sum_lo(float x) {
#pragma unroll
  for (int bit = 0; bit < HI; ++bit) x += __shfl_xor(x, 1 << bit, 64);
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
  static constexpr int NPASS = 2;
  static constexpr int T = KPP * NPASS;    // keys per wave tile
  static constexpr int LPV = D / 8;        // lanes per key, PV layout
  static constexpr int KPV = 64 / LPV;     // keys per PV step
  static constexpr int NSTEP = T / KPV;    // PV steps per tile
  static constexpr int LOG_LPK = ilog2c(LPK);
  static constexpr int LOG_LPV = ilog2c(LPV);
  static constexpr int PBUF = NW * T * RP;             // floats
  static constexpr int MERGE = NW * RP * D + NW * RP * 2;
  static constexpr int SMEM = PBUF > MERGE ? PBUF : MERGE;
};

template <int D, int RP, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(kWavesPerBlock * 64) void split_decode_valu(const DecodeArgs a) {
  using Lay = Layout<D, RP>;
  constexpr int NW = Lay::NW, LPK = Lay::LPK, KPP = Lay::KPP, NPASS = Lay::NPASS, T = Lay::T;
  constexpr int LPV = Lay::LPV, KPV = Lay::KPV, NSTEP = Lay::NSTEP;
  __shared__ __attribute__((aligned(16))) float smem[Lay::SMEM];

  // ---- unit decode (XCD-aware): siblings (kv head, row block) of one
  // (b, split) unit get consecutive slots on the same XCD
  const int x = blockIdx.x;
  const int xcd = x & 7;
  const int slot = x >> 3;
  const int inner_idx = slot % a.inner;
  const int outer_idx = (slot / a.inner) * 8 + xcd;
  if (outer_idx >= a.outer) return;
  const int b = outer_idx / a.S;
  const int s = outer_idx - b * a.S;
  const int g = inner_idx / a.nrb;
  const int rb = inner_idx - g * a.nrb;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int jq = lane / LPK, qq = lane % LPK;   // QK layout
  const int kg = lane / LPV, ds = lane % LPV;   // PV layout

  const int r0 = rb * RP;
  const int L = a.kv_lens[b];
  int c = -1;
  if (CAUSAL) c = a.causal_offsets ? a.causal_offsets[b] : a.causal_offset;

  // per-row visible key limit and the block's key range
  int lim[RP];
  int kmax = 0;
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    const int rr = r0 + r;
    int lr = 0;
    if (rr < a.R) {
      lr = L;
      if (CAUSAL && c >= 0) {
        const int64_t cl = (int64_t)c + rr / a.G + 1;
        if (cl < lr) lr = (int)cl;
      }
    }
    lim[r] = lr;
    kmax = lr > kmax ? lr : kmax;
  }
  const int kb = s * a.chunk;
  int ke = kb + a.chunk;
  if (ke > kmax) ke = kmax;
  const int ntiles = kb < ke ? (ke - kb + T - 1) / T : 0;

  // ---- q rows of this block in registers (QK layout: chunks qq + LPK*c4)
  uint32_t qr[RP][16];
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    const int rr = r0 + r;
    if (rr < a.R) {
      const int i = rr / a.G;
      const int h = g * a.G + (rr - i * a.G);
      const uint4 *src = reinterpret_cast<const uint4 *>(a.q + (((int64_t)b * a.q_len + i) * a.Hq + h) * D);
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const uint4 t = src[qq + LPK * c4];
        qr[r][4 * c4 + 0] = t.x;
        qr[r][4 * c4 + 1] = t.y;
        qr[r][4 * c4 + 2] = t.z;
        qr[r][4 * c4 + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) qr[r][e] = 0u;
    }
  }

  const int *bt_row = a.block_table + (int64_t)b * a.max_pages;
  const uint16_t *kbase = a.k + g * D;
  const uint16_t *vbase = a.v + g * D;
  const int pmask = (1 << a.page_shift) - 1;
  float *pbuf = smem + w * (T * RP);

  float m_run[RP], l_part[RP], acc[RP][8];
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    m_run[r] = -INFINITY;
    l_part[r] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
  }

  for (int t = w; t < ntiles; t += NW) {
    const int base = kb + t * T;
    // K rows, QK layout
    uint4 kr[NPASS][4];
#pragma unroll
    for (int pp = 0; pp < NPASS; ++pp) {
      const int j = base + pp * KPP + jq;
      if (j < ke) {
        const int page = bt_row[j >> a.page_shift];
        const int64_t off = (int64_t)page * a.page_stride + (int64_t)(j & pmask) * a.row_stride;
        const uint4 *src = reinterpret_cast<const uint4 *>(kbase + off);
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) kr[pp][c4] = src[qq + LPK * c4];
      } else {
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) kr[pp][c4] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    // V rows, PV layout
    uint4 vr[NSTEP];
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      const int j = base + st * KPV + kg;
      if (j < ke) {
        const int page = bt_row[j >> a.page_shift];
        const int64_t off = (int64_t)page * a.page_stride + (int64_t)(j & pmask) * a.row_stride;
        vr[st] = reinterpret_cast<const uint4 *>(vbase + off)[ds];
      } else {
        vr[st] = make_uint4(0u, 0u, 0u, 0u);
      }
    }

    // scores
    float sc[NPASS][RP];
#pragma unroll
    for (int pp = 0; pp < NPASS; ++pp) {
#pragma unroll
      for (int r = 0; r < RP; ++r) {
        float d = 0.f;
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
#pragma unroll
          for (int e = 0; e < 4; ++e) d = dot2_bf16(comp(kr[pp][c4], e), qr[r][4 * c4 + e], d);
        sc[pp][r] = wave_sum_lo<Lay::LOG_LPK>(d);
      }
    }
#pragma unroll
    for (int pp = 0; pp < NPASS; ++pp) {
      const int j = base + pp * KPP + jq;
      const bool in = j < ke;
      float mv[RP];
#pragma unroll
      for (int r = 0; r < RP; ++r) mv[r] = 0.f;
      if (MASK && in) {
        if (a.mask_sq == 0) {
          const float m0 = a.mask[(int64_t)b * a.mask_sb + j] * kLog2e;
#pragma unroll
          for (int r = 0; r < RP; ++r) mv[r] = m0;
        } else {
#pragma unroll
          for (int r = 0; r < RP; ++r) {
            const int rr = r0 + r < a.R ? r0 + r : a.R - 1;
            mv[r] = a.mask[(int64_t)b * a.mask_sb + (int64_t)(rr / a.G) * a.mask_sq + j] * kLog2e;
          }
        }
      }
#pragma unroll
      for (int r = 0; r < RP; ++r) {
        const float v = sc[pp][r] * a.scale_log2 + mv[r];
        const bool vis = CAUSAL ? (j < lim[r] && in) : (in && r0 + r < a.R);
        sc[pp][r] = vis ? v : -INFINITY;
      }
    }

    // online softmax update
    float alpha[RP], mu[RP];
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      float mt = sc[0][r];
#pragma unroll
      for (int pp = 1; pp < NPASS; ++pp) mt = fmaxf(mt, sc[pp][r]);
      mt = wave_max_hi<Lay::LOG_LPK>(mt);
      const float mnew = fmaxf(m_run[r], mt);
      const float use = mnew == -INFINITY ? 0.f : mnew;
      alpha[r] = fast_exp2(m_run[r] - use);
      m_run[r] = mnew;
      mu[r] = use;
    }
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      float lsum = 0.f;
#pragma unroll
      for (int pp = 0; pp < NPASS; ++pp) {
        const float pv = fast_exp2(sc[pp][r] - mu[r]);
        lsum += pv;
        if ((r % LPK) == qq) pbuf[(pp * KPP + jq) * RP + r] = pv;
      }
      l_part[r] = l_part[r] * alpha[r] + lsum;
    }
    __builtin_amdgcn_wave_barrier();

    // PV
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r][e] *= alpha[r];
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      const int key = st * KPV + kg;
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
      } else {
#pragma unroll
        for (int r = 0; r < RP; ++r) pr[r] = pbuf[key * RP + r];
      }
      float vf[8];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const uint32_t u = comp(vr[st], e2);
        vf[2 * e2] = bf16_lo(u);
        vf[2 * e2 + 1] = bf16_hi(u);
      }
#pragma unroll
      for (int r = 0; r < RP; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = fmaf(pr[r], vf[e], acc[r][e]);
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- wave totals: l over QK key groups, acc over PV key groups
  float l_tot[RP];
#pragma unroll
  for (int r = 0; r < RP; ++r) l_tot[r] = wave_sum_hi<Lay::LOG_LPK>(l_part[r]);
#pragma unroll
  for (int r = 0; r < RP; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = wave_sum_hi<Lay::LOG_LPV>(acc[r][e]);

  // ---- merge the waves through LDS and write
  __syncthreads();
  float *ob = smem;                    // [NW][RP][D]
  float *mlb = smem + NW * RP * D;     // [NW][RP][2]
  if (kg == 0) {
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      float4 *dst = reinterpret_cast<float4 *>(ob + (w * RP + r) * D + ds * 8);
      dst[0] = make_float4(acc[r][0], acc[r][1], acc[r][2], acc[r][3]);
      dst[1] = make_float4(acc[r][4], acc[r][5], acc[r][6], acc[r][7]);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      mlb[(w * RP + r) * 2] = m_run[r];
      mlb[(w * RP + r) * 2 + 1] = l_tot[r];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < RP * D; idx += NW * 64) {
    const int r = idx / D;
    const int d = idx - r * D;
    const int rr = r0 + r;
    if (rr >= a.R) continue;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww)
      if (mlb[(ww * RP + r) * 2 + 1] > 0.f) M = fmaxf(M, mlb[(ww * RP + r) * 2]);
    float W = 0.f, o = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float lw = mlb[(ww * RP + r) * 2 + 1];
        if (lw > 0.f) {
          const float f = fast_exp2(mlb[(ww * RP + r) * 2] - M);
          W = fmaf(f, lw, W);
          o = fmaf(f, ob[(ww * RP + r) * D + d], o);
        }
      }
    }
    const float res = W > 0.f ? o / W : 0.f;
    const int i = rr / a.G;
    const int h = g * a.G + (rr - i * a.G);
    const int64_t row = ((int64_t)b * a.q_len + i) * a.Hq + h;
    if (!a.partials) {
      a.out[row * D + d] = f32_to_bf16_rne(res);
      if (a.out_f32) a.out_f32[row * D + d] = res;
    } else {
      a.o_part[(row * a.S + s) * D + d] = res;
      if (d == 0) {
        a.ml_part[(row * a.S + s) * 2] = W > 0.f ? M * kLn2 : -INFINITY;
        a.ml_part[(row * a.S + s) * 2 + 1] = W;
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const CombineArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int lane = threadIdx.x & 63;
  constexpr int PER = (D + 63) / 64;
  const float *ml = a.ml_part + row * a.S * 2;
  const float *op = a.o_part + row * a.S * D;
  float M = -INFINITY;
  for (int s = 0; s < a.S; ++s)
    if (ml[2 * s + 1] > 0.f) M = fmaxf(M, ml[2 * s]);
  float o[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) o[k] = 0.f;
  float W = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < a.S; ++s) {
      const float l = ml[2 * s + 1];
      if (!(l > 0.f)) continue;
      const float f = l * fast_exp2((ml[2 * s] - M) * kLog2e);
      W += f;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int d = lane + 64 * k;
        if (d < D) o[k] = fmaf(f, op[s * D + d], o[k]);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int d = lane + 64 * k;
    if (d < D) {
      const float res = W > 0.f ? o[k] / W : 0.f;
      a.out[row * D + d] = f32_to_bf16_rne(res);
      if (a.out_f32) a.out_f32[row * D + d] = res;
    }
  }
}

template <int D, int RP, bool C, bool M>
hipError_t launch_t(const DecodeArgs &a, hipStream_t stream) {
  const int64_t outer_pad = ((int64_t)a.outer + 7) / 8 * 8;
  const int64_t grid = outer_pad * a.inner;
  hipLaunchKernelGGL((split_decode_valu<D, RP, C, M>), dim3((unsigned)grid), dim3(kWavesPerBlock * 64), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D, int RP>
hipError_t launch_rp(const DecodeArgs &a, bool causal, bool mask, hipStream_t s) {
  if (causal) return mask ? launch_t<D, RP, true, true>(a, s) : launch_t<D, RP, true, false>(a, s);
  return mask ? launch_t<D, RP, false, true>(a, s) : launch_t<D, RP, false, false>(a, s);
}

template <int D>
hipError_t launch_d(const DecodeArgs &a, int rp, bool causal, bool mask, hipStream_t s) {
  switch (rp) {
    case 1: return launch_rp<D, 1>(a, causal, mask, s);
    case 2: return launch_rp<D, 2>(a, causal, mask, s);
    case 4: return launch_rp<D, 4>(a, causal, mask, s);
    default: return launch_rp<D, 8>(a, causal, mask, s);
  }
}

}  // namespace

int launch_split(const DecodeArgs &a, int head_dim, int rp, bool causal, bool has_mask,
                 hipStream_t stream) {
  switch (head_dim) {
    case 32: return launch_d<32>(a, rp, causal, has_mask, stream);
    case 64: return launch_d<64>(a, rp, causal, has_mask, stream);
    case 128: return launch_d<128>(a, rp, causal, has_mask, stream);
    default: return launch_d<256>(a, rp, causal, has_mask, stream);
  }
}

int launch_combine(const CombineArgs &a, int head_dim, hipStream_t stream) {
  const unsigned grid = (unsigned)((a.rows + 3) / 4);
  switch (head_dim) {
    case 32: hipLaunchKernelGGL(combine_kernel<32>, dim3(grid), dim3(256), 0, stream, a); break;
    case 64: hipLaunchKernelGGL(combine_kernel<64>, dim3(grid), dim3(256), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(combine_kernel<128>, dim3(grid), dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL(combine_kernel<256>, dim3(grid), dim3(256), 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace pkv
