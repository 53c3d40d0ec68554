// Gather-attention for gfx950 (AB-Attention page, section "AB-Attention ve Üç
// Temel Yeniliği", third item: KV blocks much smaller than a tile are packed
// into full matrix-core tiles; SIP item: the 1/pi weights act inside the
// softmax numerator and denominator).  Dense attention is the same pipeline
// with contiguous KV tiles and unit weights.
//
// One workgroup owns one row (b, h, query block): BQ/32 waves, each holding 32
// queries.  The row's KV blocks are gathered 64 keys at a time (64/BK list
// entries per tile) from HBM into LDS.  Per tile and wave:
//   S^T = K Q^T   on v_mfma_f32_32x32x16_bf16 (A = K tile from LDS, B = the
//                 wave's queries, kept in registers for the whole row);
//   t = S * scale*log2(e) + log2(w_b)   (w_b the block's weight; -inf for
//                 keys outside the list or past L);
//   online max / exp2 / row sums per query (fp32), P rounded to bf16;
//   O^T += V^T P^T on the same MFMA (A = V^T tile from LDS, B = P^T straight
//                 from the S^T accumulators: the accumulator layout of the
//                 first product is the operand layout of the second).
// With queries in the N position of both products, each lane owns one query,
// so the softmax statistics and the O^T rescale stay in-lane.
#include "absa_device.h"
#include "absa_launch.h"

namespace absa {

// Byte offset of 16-byte chunk c of key row kk in the K tile ([64][D] bf16):
// chunks are xor-swizzled by the row so the 16 rows read by a quarter-wave hit
// 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int k_off(int kk, int c) {
  if constexpr (D == 128) return kk * 256 + ((c ^ (kk & 15)) << 4);
  else return kk * 128 + ((c ^ ((kk >> 1) & 7)) << 4);
}

// Byte offset of 8-byte unit u (keys 4u..4u+3) of row dc in the V^T tile
// ([D][64] bf16, 128 bytes per row), xor-swizzled by (dc >> 1).
__device__ __forceinline__ int vt_off(int dc, int u) { return dc * 128 + ((u ^ ((dc >> 1) & 15)) << 3); }

template <int D, int BQ, int BK, bool DENSE, bool OUT_BF16>
__global__ __launch_bounds__(BQ * 2) void attend_kernel(AttendLaunch a) {
  constexpr int NT = BQ * 2;           // BQ/32 waves of 64 lanes
  constexpr int CPR = D / 8;           // 16-byte chunks per key row
  constexpr int NCH = 64 * CPR / NT;   // chunks per thread per tile (K and V each)
  constexpr int SPT = 64 / BK;         // list entries per 64-key tile
  constexpr int KS = D / 16;           // k-steps of the QK product
  constexpr int DB = D / 32;           // 32-wide d blocks of O

  __shared__ __attribute__((aligned(16))) unsigned char k_lds[64 * D * 2];
  __shared__ __attribute__((aligned(16))) unsigned char vt_lds[64 * D * 2];
  __shared__ float bias_lds[64];

  // XCD-aware row order: workgroup w runs on XCD w % 8, so give each XCD a
  // contiguous range of rows (consecutive query blocks of the same heads share
  // their KV blocks through that XCD's L2).
  const int nper = (a.rows + 7) >> 3;
  const int row = (blockIdx.x & 7) * nper + (blockIdx.x >> 3);
  if (row >= a.rows) return;
  const int bh = row / a.NQ, qb = row % a.NQ;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int h = lane >> 5, qn = lane & 31;
  const size_t head_off = (size_t)bh * a.L * D;
  const uint16_t* __restrict__ kh = a.k + head_off;
  const uint16_t* __restrict__ vh = a.v + head_off;

  // ---- this lane's query, as the B operand of S^T = K Q^T
  const int qi = qb * BQ + wid * 32 + qn;
  bf16x8 qf[KS];
  {
    const bool qv = qi < a.L;
    const uint4* qp = reinterpret_cast<const uint4*>(a.q + head_off + (size_t)(qv ? qi : 0) * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 w = qp[2 * ks + h];
      if (!qv) w = make_uint4(0, 0, 0, 0);
      qf[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // ---- the row's list
  int nblk, ntiles;
  const int32_t* lidx = nullptr;
  const float* lw = nullptr;
  if constexpr (DENSE) {
    nblk = (a.L + BK - 1) / BK;
    ntiles = (a.L + 63) / 64;
  } else {
    nblk = a.count[row];
    nblk = nblk < 0 ? 0 : (nblk > a.cap ? a.cap : nblk);
    ntiles = (nblk + SPT - 1) / SPT;
    lidx = a.kv_idx + (size_t)row * a.cap;
    lw = a.inv_pi + (size_t)row * a.cap;
  }

  // ---- gather of one tile into registers
  uint4 kreg[NCH], vreg[NCH];
  float bias_reg = -INFINITY;
  auto gather = [&](int tile) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int g = tid + j * NT;
      const int kk = g / CPR, c = g % CPR;
      const int slot = kk / BK, r = kk % BK;
      const int e = tile * SPT + slot;
      int blk = -1;
      if constexpr (DENSE) blk = e;
      else if (e < nblk) blk = lidx[e];
      const int key = blk * BK + r;
      const bool ok = DENSE ? key < a.L : (blk >= 0 && blk < a.NK && key < a.L);
      uint4 kv4 = make_uint4(0, 0, 0, 0), vv4 = make_uint4(0, 0, 0, 0);
      if (ok) {
        kv4 = *reinterpret_cast<const uint4*>(kh + (size_t)key * D + c * 8);
        vv4 = *reinterpret_cast<const uint4*>(vh + (size_t)key * D + c * 8);
      }
      kreg[j] = kv4;
      vreg[j] = vv4;
    }
    if (tid < 64) {
      const int kk = tid, slot = kk / BK, r = kk % BK;
      const int e = tile * SPT + slot;
      float b = -INFINITY;
      if constexpr (DENSE) {
        if (e * BK + r < a.L) b = 0.f;
      } else if (e < nblk) {
        const int blk = lidx[e];
        if (blk >= 0 && blk < a.NK && blk * BK + r < a.L) b = __log2f(lw[e]);
      }
      bias_reg = b;
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int g = tid + j * NT;
      const int kk = g / CPR, c = g % CPR;
      *reinterpret_cast<uint4*>(k_lds + k_off<D>(kk, c)) = kreg[j];
      const uint32_t w[4] = {vreg[j].x, vreg[j].y, vreg[j].z, vreg[j].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dc = c * 8 + e;
        const uint16_t val = (uint16_t)((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu));
        *reinterpret_cast<uint16_t*>(vt_lds + vt_off(dc, kk >> 2) + (kk & 3) * 2) = val;
      }
    }
    if (tid < 64) bias_lds[tid] = bias_reg;
  };

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale_log2;

  if (ntiles > 0) gather(0);
#pragma unroll 1
  for (int tile = 0; tile < ntiles; ++tile) {
    __syncthreads();
    stash();
    __syncthreads();
    if (tile + 1 < ntiles) gather(tile + 1);

    // S^T for 64 keys (two 32-key halves) x this wave's 32 queries
    f32x16 sacc[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[sb][r] = 0.f;
      const int kk = sb * 32 + qn;  // A-operand row (key) of this lane
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 kfrag = *reinterpret_cast<const bf16x8*>(k_lds + k_off<D>(kk, 2 * ks + h));
        sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag, qf[ks], sacc[sb], 0, 0, 0);
      }
    }
    // lane (h, qn) register r of half sb holds key 32 sb + 8 (r/4) + 4 h + r%4
    float mt = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = sb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const float tv = fmaf(sacc[sb][r], sl2, bias_lds[kk]);
        sacc[sb][r] = tv;
        mt = fmaxf(mt, tv);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    bf16x8 pf[4];
    float psum = 0.f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(sacc[sb][half * 8 + e] - m_use);
          const __bf16 pb = (__bf16)p;
          pf[sb * 2 + half][e] = pb;
          psum += (float)pb;
        }
    l_run = fmaf(l_run, alpha, psum);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;

    // O^T += V^T P^T: k-step ks covers keys 16 ks .. 16 ks + 15; this lane's 8
    // keys are 16 ks + {4h..4h+3} and 16 ks + 8 + {4h..4h+3}, matching pf[ks].
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int dc = db * 32 + qn;
        const uint2 lo = *reinterpret_cast<const uint2*>(vt_lds + vt_off(dc, 4 * ks + h));
        const uint2 hi = *reinterpret_cast<const uint2*>(vt_lds + vt_off(dc, 4 * ks + 2 + h));
        const uint4 w = make_uint4(lo.x, lo.y, hi.x, hi.y);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pf[ks],
                                                          acc[db], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: O = O^T / l, valid queries only
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (qi < a.L) {
    const size_t obase = head_off + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dc = db * 32 + 8 * g4 + 4 * h;
        const float o0 = acc[db][4 * g4 + 0] * inv, o1 = acc[db][4 * g4 + 1] * inv;
        const float o2 = acc[db][4 * g4 + 2] * inv, o3 = acc[db][4 * g4 + 3] * inv;
        if constexpr (OUT_BF16) {
          const __bf16 b0 = (__bf16)o0, b1 = (__bf16)o1, b2 = (__bf16)o2, b3 = (__bf16)o3;
          const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, b0) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
          const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, b2) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.o) + obase + dc) = make_uint2(w0, w1);
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.o) + obase + dc) =
              make_float4(o0, o1, o2, o3);
        }
      }
  }
}

// ============================================================================= launchers
template <int D, int BQ, int BK, bool DENSE>
static hipError_t launch_t(const AttendLaunch& a, hipStream_t st) {
  const int nper = (a.rows + 7) / 8;
  dim3 grid(nper * 8);
  if (a.out_bf16)
    attend_kernel<D, BQ, BK, DENSE, true><<<grid, BQ * 2, 0, st>>>(a);
  else
    attend_kernel<D, BQ, BK, DENSE, false><<<grid, BQ * 2, 0, st>>>(a);
  return hipGetLastError();
}

template <int D, int BQ>
static hipError_t launch_bk(const AttendLaunch& a, hipStream_t st, bool dense) {
  if (dense) return launch_t<D, BQ, 64, true>(a, st);
  switch (a.Bk) {
    case 16: return launch_t<D, BQ, 16, false>(a, st);
    case 32: return launch_t<D, BQ, 32, false>(a, st);
    default: return launch_t<D, BQ, 64, false>(a, st);
  }
}

hipError_t launch_attend(const AttendLaunch& a, hipStream_t st, bool dense) {
  if (a.d == 128) {
    return a.Bq == 128 ? launch_bk<128, 128>(a, st, dense) : launch_bk<128, 64>(a, st, dense);
  }
  return a.Bq == 128 ? launch_bk<64, 128>(a, st, dense) : launch_bk<64, 64>(a, st, dense);
}

}  // namespace absa
