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

template <int D, int BQ, int BK, bool DENSE, bool OUT_BF16>
__global__ __launch_bounds__(BQ * 2, 512 / (BQ * 2)) void attend_kernel(AttendLaunch a) {
  constexpr int NT = BQ * 2;           // BQ/32 waves of 64 lanes
  constexpr int CPR = D / 8;           // 16-byte chunks per key row
  constexpr int NCH = 64 * CPR / NT;   // chunks per thread per tile (K and V each)
  constexpr int SPT = 64 / BK;         // list entries per 64-key tile
  constexpr int KS = D / 16;           // k-steps of the QK product
  constexpr int DB = D / 32;           // 32-wide d blocks of O
  constexpr int TILE = 64 * D * 2;     // bytes of one K or V tile
  // Rescale threshold (log2 units): the running max is only moved when a
  // tile's max exceeds it by more than this, so P stays <= 2^8.
  constexpr float TAU = 8.f;

  __shared__ __attribute__((aligned(16))) unsigned char k_lds[2][TILE];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds[2][TILE];
  __shared__ __attribute__((aligned(16))) float bias_lds[2][64];
  __shared__ int tail_lds[2];

  // Row order.  Workgroups are dealt round-robin over the 8 XCDs, so a run of
  // 8*64 consecutive workgroups covers ~one head's worth of rows that all share
  // that head's K/V in the last-level cache.  Within such a group, XCD x takes
  // the 64 adjacent query blocks [64x, 64x+64): neighbouring query blocks of a
  // video select overlapping KV blocks, which then hit in that XCD's L2.
  int row = blockIdx.x;
  {
    constexpr int R = 64, S = 8 * R;
    const int g = row / S, i = row % S;
    if ((g + 1) * S <= a.rows) row = g * S + (i & 7) * R + (i >> 3);
  }
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

  // ---- gather of one tile into registers, and their store into an LDS buffer.
  // The list entries a tile needs are fetched one iteration before its K/V
  // loads are issued, so no K/V load waits on a list load.  K/V loads are
  // unconditional: a masked key reads row 0 of the head (in bounds, finite) and
  // its -inf bias removes it from the softmax.
  // Raw list entries: *_cur for the tile whose K/V loads are issued next,
  // *_nxt for the one after.  The loads of *_nxt are issued before the K/V loads
  // and only read an iteration later (memory waits retire in issue order, so a
  // list load issued after the K/V loads would hold them up).
  int nb_cur[NCH], nb_nxt[NCH];
  int nbb_cur = 0, nbb_nxt = 0;        // threads 0..63: block of key `tid`
  float nbw_cur = 1.f, nbw_nxt = 1.f;  // and its weight
  auto fetch_idx = [&](int tile) {     // raw entries of `tile` into *_nxt
    if constexpr (!DENSE) {
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int e = tile * SPT + ((tid + j * NT) / CPR) / BK;
        const int ec = e < nblk ? e : nblk - 1;
        nb_nxt[j] = lidx[ec < 0 ? 0 : ec];
      }
      if (tid < 64) {
        const int e = tile * SPT + tid / BK;
        const int ec = e < nblk ? e : nblk - 1;
        nbb_nxt = lidx[ec < 0 ? 0 : ec];
        nbw_nxt = lw[ec < 0 ? 0 : ec];
      }
    }
  };
  auto rotate_idx = [&]() {
#pragma unroll
    for (int j = 0; j < NCH; ++j) nb_cur[j] = nb_nxt[j];
    nbb_cur = nbb_nxt;
    nbw_cur = nbw_nxt;
  };
  u32x4 kreg[NCH], vreg[NCH];
  float bias_reg = -INFINITY;
  bool tail_reg = false;
  auto gather = [&](int tile) {  // K/V loads of `tile`, whose entries are in *_cur
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int g = tid + j * NT;
      const int kk = g / CPR, c = g % CPR;
      const int r = kk % BK;
      const int e = tile * SPT + kk / BK;
      const int blk = DENSE ? e : (e < nblk ? nb_cur[j] : -1);
      const int key = blk * BK + r;
      const bool ok = DENSE ? key < a.L : (blk >= 0 && blk < a.NK && key < a.L);
      const size_t off = (size_t)(ok ? key : 0) * D + c * 8;
      kreg[j] = *reinterpret_cast<const u32x4*>(kh + off);
      vreg[j] = *reinterpret_cast<const u32x4*>(vh + off);
    }
    if (tid < 64) {
      const int e = tile * SPT + tid / BK;
      const int blk = DENSE ? e : (e < nblk ? nbb_cur : -1);
      const int key = blk * BK + tid % BK;
      const bool slot_ok = DENSE ? true : (blk >= 0 && blk < a.NK);
      bias_reg = (slot_ok && key < a.L) ? (DENSE ? 0.f : __log2f(nbw_cur)) : -INFINITY;
      tail_reg = slot_ok && key >= a.L;  // a key past L inside a listed block
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int g = tid + j * NT;
      const int kk = g / CPR, c = g % CPR;
      *reinterpret_cast<u32x4*>(&k_lds[buf][k_off<D>(kk, c)]) = kreg[j];
      *reinterpret_cast<u32x4*>(&v_lds[buf][v_off<D>(kk, c)]) = vreg[j];
    }
    if (wid == 0) {
      bias_lds[buf][lane] = bias_reg;
      const unsigned long long any_tail = __ballot(tail_reg);
      if (lane == 0) tail_lds[buf] = any_tail != 0ull;
    }
  };

  // ---- per-lane offsets of the transposing V reads (see v_off): 16-lane group
  // G, lane s in it; source row 4h + s/4 (+16 ks + 8 j), columns 32 db + 16 (G&1)
  // + 4 (s&3) .. +3.
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

  if (ntiles > 0) {
    fetch_idx(0);
    rotate_idx();
    if (ntiles > 1) fetch_idx(1);
    gather(0);
    stash(0);
    rotate_idx();
  }
#pragma unroll 1
  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    __syncthreads();  // tile is in buf; every wave is done with buf ^ 1
    if (tile + 2 < ntiles) fetch_idx(tile + 2);  // list entries of tile + 2 (first)
    if (tile + 1 < ntiles) gather(tile + 1);     // K/V of tile + 1
    const unsigned char* kb = k_lds[buf];
    const unsigned char* vb = v_lds[buf];

    // S^T for 64 keys (two 32-key halves) x this wave's 32 queries
    f32x16 sacc[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[sb][r] = 0.f;
      const int kk = sb * 32 + qn;  // A-operand row (key) of this lane
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 kfrag = *reinterpret_cast<const bf16x8*>(kb + k_off<D>(kk, 2 * ks + h));
        sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag, qf[ks], sacc[sb], 0, 0, 0);
      }
    }
    // Lane (h, qn) register r of half sb holds key 32 sb + 8 (r/4) + 4 h + r%4.
    // t = S scale log2(e) + log2(w_block) - m, with m the running reference.
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float mt = -INFINITY;
    if (!tail_lds[buf]) {
      // every 4-key group lies in one block and is all valid or all masked
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float cg = bias_lds[buf][32 * sb + 8 * g4 + 4 * h] - m_use;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float tv = fmaf(sacc[sb][4 * g4 + i], sl2, cg);
            sacc[sb][4 * g4 + i] = tv;
            mt = fmaxf(mt, tv);
          }
        }
    } else {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = sb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          const float tv = fmaf(sacc[sb][r], sl2, bias_lds[buf][kk] - m_use);
          sacc[sb][r] = tv;
          mt = fmaxf(mt, tv);
        }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    // Move the reference only when needed (first valid tile, or growth > TAU).
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
    // P = 2^t rounded to bf16; the row sum adds exactly these rounded values
    bf16x8 pf[4];
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

    // O^T += V^T P^T: k-step ks covers keys 16 ks .. 16 ks + 15; this lane's 8
    // keys are 16 ks + {4h..4h+3} and 16 ks + 8 + {4h..4h+3}, matching pf[ks];
    // the two transposing reads deliver exactly those keys for column 32 db + qn.
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
        const unsigned char* p0 = vb + voff[db] + (16 * ks) * (D * 2);
        const unsigned char* p1 = p0 + 8 * (D * 2);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
        const i16x4 w[2] = {lo, hi};
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pf[ks],
                                                          acc[db], 0, 0, 0);
      }
    }
    if (tile + 1 < ntiles) stash(buf ^ 1);
    rotate_idx();
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
