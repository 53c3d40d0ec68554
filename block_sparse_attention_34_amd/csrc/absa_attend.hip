// Gather-attention for gfx950 (AB-Attention page, section "AB-Attention ve Üç
// Temel Yeniliği", third item: KV blocks much smaller than a tile are packed
// into full matrix-core tiles; SIP item: the 1/pi weights act inside the
// softmax numerator and denominator).  Dense attention is the same pipeline
// with contiguous KV tiles and unit weights.
//
// One workgroup owns one row (b, h, query block): BQ/32 waves, each holding 32
// queries.  The row's KV blocks are gathered 64 keys at a time (64/BK list
// entries per tile) from HBM straight into LDS.  Per tile and wave:
//   S^T = K Q^T   on v_mfma_f32_32x32x16_bf16 (A = K tile from LDS, B = the
//                 wave's queries, kept in registers for the whole row);
//   t = S * scale*log2(e) + log2(w_b)   (w_b the block's weight; -inf for
//                 keys outside the list or past L);
//   online max / exp2 / row sums per query (fp32), P rounded to bf16;
//   O^T += V^T P^T on the same MFMA (A = V^T read transposed from the
//                 row-major V tile with ds_read_b64_tr_b16, B = P^T straight
//                 from the S^T accumulators: the accumulator layout of the
//                 first product is the operand layout of the second).
// With queries in the N position of both products, each lane owns one query,
// so the softmax statistics and the O^T rescale stay in-lane.  The tiles of
// tile n+1 load while tile n computes (two LDS slots, one barrier per tile).
#include <type_traits>

#include "absa_device.h"
#include "absa_launch.h"

namespace absa {

// LDS tiles hold 64 keys x D bf16 row-major, 16-byte chunks xor-swizzled by row.
// K tile: chunk c of row kk at c ^ (kk & 15) (D = 128) so that the 16 rows read
// by a quarter-wave (one 16-byte chunk each) hit distinct bank groups.
template <int D>
__device__ __forceinline__ int k_off(int kk, int c) {
  if constexpr (D == 128) return kk * 256 + ((c ^ (kk & 15)) << 4);
  else return kk * 128 + ((c ^ ((kk >> 1) & 7)) << 4);
}

// V tile: chunk c of row kk at c ^ 2(kk & 7) (D = 128).  V is read with
// ds_read_b64_tr_b16, where a 16-lane group reads 4 consecutive rows x 32
// bytes; the even xor keeps those 8 chunks on distinct bank groups.
template <int D>
__device__ __forceinline__ int v_off(int kk, int c) {
  if constexpr (D == 128) return kk * 256 + ((c ^ ((kk & 7) << 1)) << 4);
  else return kk * 128 + ((c ^ ((kk & 3) << 1)) << 4);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // a first-class vector, kept in VGPRs

// K and V tiles arrive by direct global->LDS loads (global_load_lds_dwordx4:
// lane l of a wave writes LDS base + 16 l), so no registers or LDS-store
// instructions stage them; the row swizzle is applied by choosing which global
// chunk each lane fetches.  The tile loop is unrolled by two so both ring slots
// are distinct static LDS arrays.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

template <int D, int BQ, int BK, bool DENSE, bool OUT_BF16>
__global__ __launch_bounds__(BQ * 2, 512 / (BQ * 2)) void attend_kernel(AttendLaunch a) {
  constexpr int NT = BQ * 2;           // threads
  constexpr int NW = BQ / 32;          // waves, 32 queries each
  constexpr int CPR = D / 8;           // 16-byte chunks per key row
  constexpr int KPI = 64 / CPR;        // key rows covered by one wave-wide 16-byte load
  constexpr int NCH = 64 * CPR / NT;   // wave-wide loads per thread per tile and tensor
  constexpr int SPT = 64 / BK;         // list entries per 64-key tile
  constexpr int KS = D / 16;           // k-steps of the QK product
  constexpr int DB = D / 32;           // 32-wide d blocks of O
  constexpr int TILE = 64 * D * 2;
  constexpr float TAU = 8.f;

  __shared__ __attribute__((aligned(16))) unsigned char k_s0[TILE];
  __shared__ __attribute__((aligned(16))) unsigned char k_s1[TILE];
  __shared__ __attribute__((aligned(16))) unsigned char v_s0[TILE];
  __shared__ __attribute__((aligned(16))) unsigned char v_s1[TILE];
  __shared__ __attribute__((aligned(16))) float bias_s[2][64];
  __shared__ int tail_s[2];

  int row = blockIdx.x;
  {
    constexpr int R = 64, S = 8 * R;
    const int g = row / S, i = row % S;
    if ((g + 1) * S <= a.rows) row = g * S + (i & 7) * R + (i >> 3);
  }
  if (row >= a.rows) return;
  const int bh = row / a.NQ, qb = row % a.NQ;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, qn = lane & 31;
  const size_t head_off = (size_t)bh * a.L * D;
  const uint16_t* __restrict__ kh = a.k + head_off;
  const uint16_t* __restrict__ vh = a.v + head_off;

  const int qi = qb * BQ + wid * 32 + qn;
  bf16x8 qf[KS];
  {
    const bool qv = qi < a.L;
    const u32x4* qp = reinterpret_cast<const u32x4*>(a.q + head_off + (size_t)(qv ? qi : 0) * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 w = qp[2 * ks + h];
      if (!qv) w = u32x4{0u, 0u, 0u, 0u};
      qf[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }

  int nblk, T;
  const int32_t* lidx = nullptr;
  const float* lw = nullptr;
  if constexpr (DENSE) {
    nblk = (a.L + BK - 1) / BK;
    T = (a.L + 63) / 64;
  } else {
    nblk = a.count[row];
    nblk = nblk < 0 ? 0 : (nblk > a.cap ? a.cap : nblk);
    T = (nblk + SPT - 1) / SPT;
    lidx = a.kv_idx + (size_t)row * a.cap;
    lw = a.inv_pi + (size_t)row * a.cap;
  }
  if (T == 0) {
    // empty list: the estimate is 0
    if (qi < a.L) {
#pragma unroll
      for (int c = 0; c < D; c += 4) {
        if constexpr (OUT_BF16)
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.o) + head_off + (size_t)qi * D + c) =
              make_uint2(0, 0);
        else
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.o) + head_off + (size_t)qi * D + c) =
              make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    return;
  }

  // ---- list entries.  A wave-wide direct load covers KPI (<= BK) consecutive
  // key rows, which lie in one block, so the entry it needs is wave-uniform.
  // It is fetched with a vector load (a scalar load would share the LDS wait
  // counter and, returning out of order, stall every LDS wait behind it) and
  // made uniform when used.  Set F is fetched for tile n+3 during iteration n,
  // used for K of n+3 in iteration n+1 and for V of n+3 in n+2.
  static_assert(BK % KPI == 0, "a wave-wide load must stay inside one block");
  struct Entries {
    int blk[NCH];  // wave-uniform block index of each wave-wide load
    int bblk;      // threads 0..63: block of key `tid`
    float bw;      //               and its weight
  };
  auto fetch = [&](Entries& E, int tile) {
    if constexpr (!DENSE) {
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int kk = (j * NW + (tid >> 6)) * KPI + lane / CPR;  // same block for the whole wave
        const int e = tile * SPT + kk / BK;
        const int ec = e < nblk ? e : nblk - 1;
        E.blk[j] = lidx[ec];
      }
      if (tid < 64) {
        const int e = tile * SPT + tid / BK;
        const int ec = e < nblk ? e : nblk - 1;
        E.bblk = lidx[ec];
        E.bw = lw[ec];
      }
    }
  };
  // wave-wide direct loads of one tile of K or V (SWZ: 0 = K layout, 1 = V layout)
  auto dma = [&](const uint16_t* __restrict__ src, unsigned char* buf, const Entries& E, int tile,
                 auto SWZ) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int ii = j * NW + wid;                 // wave-wide load index: LDS positions [64 ii, 64 ii + 64)
      const int kk = ii * KPI + lane / CPR;        // key row of this lane's position
      const int cp = lane % CPR;                   // chunk position within the row
      int c;
      if constexpr (decltype(SWZ)::value == 0) c = (D == 128) ? (cp ^ (kk & 15)) : (cp ^ ((kk >> 1) & 7));
      else c = (D == 128) ? (cp ^ ((kk & 7) << 1)) : (cp ^ ((kk & 3) << 1));
      const int e = tile * SPT + (ii * KPI) / BK;
      int blk;
      if constexpr (DENSE) blk = e;
      else blk = e < nblk ? __builtin_amdgcn_readfirstlane(E.blk[j]) : -1;
      const bool blk_ok = DENSE ? true : (blk >= 0 && blk < a.NK);
      const int key = blk * BK + kk % BK;
      const bool ok = blk_ok && key < a.L;
      const uint16_t* g = src + (size_t)(ok ? key : 0) * D + c * 8;
      __builtin_amdgcn_global_load_lds((glb_void_t*)g, (lds_void_t*)(buf + ii * 1024), 16, 0, 0);
    }
  };
  auto put_bias = [&](int slot, const Entries& E, int tile) {
    if (tid < 64) {
      const int e = tile * SPT + tid / BK;
      const int blk = DENSE ? e : (e < nblk ? E.bblk : -1);
      const int key = blk * BK + tid % BK;
      const bool slot_ok = DENSE ? true : (blk >= 0 && blk < a.NK);
      bias_s[slot][tid] = (slot_ok && key < a.L) ? (DENSE ? 0.f : __log2f(E.bw)) : -INFINITY;
      const unsigned long long any_tail = __ballot(slot_ok && key >= a.L);
      if (lane == 0) tail_s[slot] = any_tail != 0ull;
    }
  };

  // V^T transposing-read offsets (see v_off)
  int voff[DB];
  {
    const int G = lane >> 4, s = lane & 15;
    const int r0 = 4 * h + (s >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int col = 32 * db + 16 * (G & 1) + 4 * (s & 3);
      voff[db] = v_off<D>(r0, col >> 3) + (col & 7) * 2;
    }
  }
  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = k_off<D>(qn, 2 * ks + h);  // rows qn and 32 + qn share it

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale_log2;
  bf16x2 ones;
  ones[0] = (__bf16)1.f;
  ones[1] = (__bf16)1.f;

  auto qk = [&](const unsigned char* kb, f32x16 (&sacc)[2]) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[sb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 kfrag = *reinterpret_cast<const bf16x8*>(kb + sb * 32 * (D * 2) + koff[ks]);
        sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag, qf[ks], sacc[sb], 0, 0, 0);
      }
    }
  };
  // Logits of one tile: t = S scale log2(e) + log2(w) - m, with the bias read
  // once per 4-key group (a group always lies in one block).  Returns this
  // lane's max.  Branch-free, so it schedules together with the next tile's QK.
  auto logits = [&](f32x16 (&sacc)[2], int slot, float m_use) {
    float mt = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const float cg = bias_s[slot][32 * sb + 8 * g4 + 4 * h] - m_use;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float tv = fmaf(sacc[sb][4 * g4 + i], sl2, cg);
          sacc[sb][4 * g4 + i] = tv;
          mt = fmaxf(mt, tv);
        }
      }
    return mt;
  };
  // Tiles holding keys past L inside a listed block (at most one per row):
  // mask those keys individually and recompute the max.
  auto mask_tail = [&](f32x16 (&sacc)[2], int slot) {
    float mt = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = sb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (bias_s[slot][kk] == -INFINITY) sacc[sb][r] = -INFINITY;
        mt = fmaxf(mt, sacc[sb][r]);
      }
    return mt;
  };
  // Rest of the softmax: move the reference if needed, P = 2^t in bf16, row sum.
  auto finish_softmax = [&](f32x16 (&sacc)[2], float mt, float m_use, bf16x8 (&pf)[4]) {
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    if (mt > TAU || (m_run == -INFINITY && mt > -INFINITY)) {
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(-mt);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      m_run = m_use + mt;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[sb][r] -= mt;
    }
    float psum = 0.f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          bf16x2 pk;
          pk[0] = (__bf16)__builtin_amdgcn_exp2f(sacc[sb][half * 8 + e]);
          pk[1] = (__bf16)__builtin_amdgcn_exp2f(sacc[sb][half * 8 + e + 1]);
          psum = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, psum, false);
          pf[sb * 2 + half][e] = pk[0];
          pf[sb * 2 + half][e + 1] = pk[1];
        }
    l_run += psum;
  };
  auto pv = [&](const unsigned char* vb, const bf16x8 (&pf)[4]) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const unsigned char* p0 = vb + voff[db] + (16 * ks) * (D * 2);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + 8 * (D * 2)));
        const i16x4 w[2] = {lo, hi};
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pf[ks],
                                                          acc[db], 0, 0, 0);
      }
    }
  };
  auto wait_dma_and_sync = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's direct loads have landed
    __syncthreads();
  };

  // ---- schedule: slot p = n % 2 holds K, V and bias of tile n; the direct
  // loads of tile n+1 into slot p^1 are issued before the compute of tile n
  // and waited for at its end, followed by one barrier.
  auto uniformize = [&](Entries& E) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) E.blk[j] = __builtin_amdgcn_readfirstlane(E.blk[j]);
  };
  Entries EC, EF;  // EC: entries of the tile whose loads are issued next; EF: being fetched
  fetch(EC, 0);
  if (T > 1) fetch(EF, 1);
  uniformize(EC);
  dma(kh, k_s0, EC, 0, std::integral_constant<int, 0>{});
  dma(vh, v_s0, EC, 0, std::integral_constant<int, 1>{});
  put_bias(0, EC, 0);
  wait_dma_and_sync();
  EC = EF;
  uniformize(EC);
  auto iteration = [&](int n, auto PAR) {
    constexpr int p = decltype(PAR)::value;
    unsigned char* k_cur = p ? k_s1 : k_s0;
    unsigned char* v_cur = p ? v_s1 : v_s0;
    unsigned char* k_nxt = p ? k_s0 : k_s1;
    unsigned char* v_nxt = p ? v_s0 : v_s1;
    if (n + 2 < T) fetch(EF, n + 2);
    if (n + 1 < T) {
      dma(kh, k_nxt, EC, n + 1, std::integral_constant<int, 0>{});
      dma(vh, v_nxt, EC, n + 1, std::integral_constant<int, 1>{});
      put_bias(p ^ 1, EC, n + 1);
    }
    f32x16 sacc[2];
    qk(k_cur, sacc);
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float mt = logits(sacc, p, m_use);
    if (tail_s[p]) mt = mask_tail(sacc, p);
    bf16x8 pf[4];
    finish_softmax(sacc, mt, m_use, pf);
    pv(v_cur, pf);
    wait_dma_and_sync();
    EC = EF;
    uniformize(EC);
  };
#pragma unroll 1
  for (int n = 0; n < T; n += 2) {
    iteration(n, std::integral_constant<int, 0>{});
    if (n + 1 < T) iteration(n + 1, std::integral_constant<int, 1>{});
  }

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
  dim3 grid(a.rows);
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
