// Gather-attention for gfx950 (AB-Attention page, section "AB-Attention ve Üç
// Temel Yeniliği", third item: KV blocks much smaller than a tile are packed
// into full matrix-core tiles; SIP item: the 1/pi weights act inside the
// softmax numerator and denominator).  Dense attention is the same pipeline
// with contiguous KV tiles and unit weights.
//
// One workgroup owns one row (b, h, query block): BQ/32 waves, each holding 32
// queries.  The row's KV blocks are gathered 64 keys at a time (64/BK list
// entries per tile; a 128-key block is two tiles) from HBM straight into LDS.  Per tile and wave:
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

#include "absa_attend_tiles.h"
#include "absa_device.h"
#include "absa_launch.h"

namespace absa {

// K, V and the per-key bias have separate two-slot LDS rings; K and the bias
// run one tile ahead of V.  Iteration n overlaps the two matrix products with
// the vector work of the neighbouring tile:
//   phase A: QK(n+1) on the matrix core  ||  2^t, bf16 rounding, row sum of tile n
//   phase B: PV(n) on the matrix core    ||  logits t of tile n+1
// then (rarely) the tail mask and the rescale of tile n+1, and one barrier.
// Tiles arrive by direct buffer->LDS loads (buffer_load_dwordx4 ... lds: lane
// l of a wave writes LDS base + 16 l); the row swizzle is applied by choosing
// which chunk each lane fetches.  The loop is unrolled by two so every ring
// slot is a distinct static LDS array.

// Two workgroups per CU hide the barrier of one behind the matrix work of the
// other; the second bound is the minimum number of waves per SIMD that allows
// them (two workgroups of BQ/32 waves over 4 SIMDs).
template <int D, int BQ, int BK, bool DENSE, bool OUT_BF16>
__global__ __launch_bounds__(BQ * 2, BQ / 64) void attend_kernel(AttendLaunch a) {
  constexpr int NT = BQ * 2;           // threads
  constexpr int NW = BQ / 32;          // waves, 32 queries each
  constexpr int CPR = D / 8;           // 16-byte chunks per key row
  constexpr int KPI = 64 / CPR;        // key rows covered by one wave-wide 16-byte load
  constexpr int NCH = 64 * CPR / NT;   // wave-wide loads per thread per tile and tensor
  constexpr int SPT = BK >= 64 ? 1 : 64 / BK;  // list entries per 64-key tile
  constexpr int TPE = BK > 64 ? BK / 64 : 1;   // 64-key tiles per list entry (128-key blocks: 2)
  constexpr int KS = D / 16;           // k-steps of the QK product
  constexpr int DB = D / 32;           // 32-wide d blocks of O
  constexpr int TILE = 64 * D * 2;
  constexpr float TAU = 8.f;           // the running max moves only when exceeded by this
  static_assert(BK % KPI == 0, "a wave-wide load must stay inside one block");
  static_assert(BK <= 64 || BK % 64 == 0, "a block larger than a tile spans whole tiles");
  static_assert(!(DENSE && BK != 64), "the dense path walks 64-key tiles");
  // list entry of key k (0..63) of a tile, and that key's row inside its block
  auto entry_of = [](int tile, int k) { return TPE > 1 ? tile / TPE : tile * SPT + k / BK; };
  auto row_in_block = [](int tile, int k) { return TPE > 1 ? (tile % TPE) * 64 + k : k % BK; };

  __shared__ __attribute__((aligned(16))) unsigned char k_s0[TILE];
  __shared__ __attribute__((aligned(16))) unsigned char k_s1[TILE];
  __shared__ __attribute__((aligned(16))) unsigned char v_s0[TILE];
  __shared__ __attribute__((aligned(16))) unsigned char v_s1[TILE];
  __shared__ __attribute__((aligned(16))) float bias_s[2][64];
  __shared__ int tail_s[2];

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
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, qn = lane & 31;
  const size_t head_off = (size_t)bh * a.L * D;

  // ---- this lane's query, as the B operand of S^T = K Q^T
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

  // ---- the row's list
  int nblk, T;
  const int32_t* lidx = nullptr;
  const float* lw = nullptr;
  if constexpr (DENSE) {
    nblk = (a.L + BK - 1) / BK;
    T = (a.L + 63) / 64;
  } else {
    nblk = a.count[row];
    nblk = nblk < 0 ? 0 : (nblk > a.cap ? a.cap : nblk);
    T = TPE > 1 ? nblk * TPE : (nblk + SPT - 1) / SPT;
    lidx = a.kv_idx + (size_t)row * a.cap;
    lw = a.inv_pi + (size_t)row * a.cap;
  }
  if (T == 0) {  // empty list: the estimate is 0
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

  // ---- direct loads.  Buffer resources cover this head's K and V (L*D*2
  // bytes); a lane's offset is a per-lane constant (row within the block,
  // swizzled chunk) plus the block's wave-uniform base.  Rows past L lie past
  // the end of the resource and entries outside the list get a base past it:
  // such loads land zeros.
  const uint32_t head_bytes = (uint32_t)a.L * D * 2;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + head_off), 0, (int)head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.v + head_off), 0, (int)head_bytes, 0x00020000);
  constexpr uint32_t OOB = 0x7FFFFFF0u;
  uint32_t klane[NCH], vlane[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int ii = j * NW + wid;
    const int kk = ii * KPI + lane / CPR, cp = lane % CPR;
    const int ck = k_chunk<D>(kk, cp), cv = v_chunk<D>(kk, cp);
    klane[j] = (uint32_t)((kk % BK) * D * 2 + ck * 16);
    vlane[j] = (uint32_t)((kk % BK) * D * 2 + cv * 16);
  }
  // List entries.  A wave-wide load covers KPI (<= BK) rows of one block, so
  // its entry is wave-uniform.  They are fetched one iteration ahead with
  // vector loads (scalar loads would share the LDS wait counter), always
  // (indices clamped to the list) so the destination registers are reused in
  // place, and consumed after the barrier that ends the iteration.
  struct Entries {
    int blk[NCH];
    int bblk;   // lane i: block of key i of the tile
    float bw;   //         and its weight
  };
  auto fetch = [&](Entries& E, int tile) {
    if constexpr (!DENSE) {
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int e = entry_of(tile, (j * NW + wid) * KPI);
        E.blk[j] = lidx[e < nblk ? e : nblk - 1];
      }
      const int e = entry_of(tile, lane);
      const int ec = e < nblk ? e : nblk - 1;
      E.bblk = lidx[ec];
      E.bw = lw[ec];
    }
  };
  // wave-uniform byte base of each wave-wide load of `tile`
  auto bases = [&](const Entries& E, int tile, uint32_t (&base)[NCH]) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int e = entry_of(tile, (j * NW + wid) * KPI);
      if constexpr (DENSE) {
        base[j] = (uint32_t)e * (BK * D * 2);
      } else {
        const int blk = __builtin_amdgcn_readfirstlane(E.blk[j]);
        const bool ok = e < nblk && blk >= 0 && blk < a.NK;
        // (a block of several tiles: this tile's keys start (tile % TPE) * 64 rows into it)
        base[j] = ok ? (uint32_t)blk * (BK * D * 2) + (uint32_t)(row_in_block(tile, 0) * D * 2) : OOB;
      }
    }
  };
  auto dma = [&](const __amdgpu_buffer_rsrc_t& rs, const uint32_t (&lanec)[NCH], const uint32_t (&base)[NCH],
                 unsigned char* buf) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      // (a named offset: an arithmetic expression in this argument position
      // makes clang's host pass drop the kernel's launch stub)
      const int off = (int)(lanec[j] + base[j]);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(buf + (j * NW + wid) * 1024), 16, off, 0, 0, 0);
    }
  };
  auto put_bias = [&](int slot, const Entries& E, int tile) {
    if (tid < 64) {
      const int e = entry_of(tile, tid);
      const int blk = DENSE ? e : E.bblk;
      const bool ok = DENSE ? true : (e < nblk && blk >= 0 && blk < a.NK);
      const int key = blk * BK + row_in_block(tile, tid);
      bias_s[slot][tid] = (ok && key < a.L) ? (DENSE ? 0.f : __log2f(E.bw)) : -INFINITY;
      const unsigned long long any_tail = __ballot(ok && key >= a.L);
      if (lane == 0) tail_s[slot] = any_tail != 0ull;
    }
  };
  auto wait_dma_and_sync = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's direct loads have landed
    __syncthreads();
  };

  // ---- per-lane LDS read offsets
  int voff[DB];  // V^T transposing reads (see v_off): 16-lane group G, lane s in it
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

  auto qk = [&](const unsigned char* kb, f32x16 (&sacc)[2]) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[sb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const bf16x8 kfrag = *reinterpret_cast<const bf16x8*>(kb + k_off<D>(sb * 32 + qn, 2 * ks + h));
        sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag, qf[ks], sacc[sb], 0, 0, 0);
      }
  };
  // t = S scale log2(e) + log2(w) - m, bias read once per 4-key group (a group
  // always lies in one block); returns this lane's max
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
  // tiles with keys past L inside a listed block (at most one per row): mask
  // those keys individually and recompute the max
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
  // move the reference when a tile exceeds it by more than TAU (or on the first
  // valid tile); afterwards sacc holds t relative to m_run
  auto rescale = [&](f32x16 (&sacc)[2], float mt, float m_use) {
    mt = half_swap_max(mt);
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
  };
  // P = 2^t rounded to bf16 in the PV operand layout; returns the row sum of
  // exactly these rounded values
  auto probs = [&](f32x16 (&sacc)[2], bf16x8 (&pf)[4]) {
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
    return psum;
  };
  auto pv = [&](const unsigned char* vb, const bf16x8 (&pf)[4]) {
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

  // ---- prologue: zeroed slots, then K(0), bias(0), V(0), K(1), bias(1);
  // S(0) = QK(0) and its logits
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int o = tid * 16; o < TILE; o += NT * 16) {
      *reinterpret_cast<u32x4*>(k_s0 + o) = z;
      *reinterpret_cast<u32x4*>(k_s1 + o) = z;
      *reinterpret_cast<u32x4*>(v_s0 + o) = z;
      *reinterpret_cast<u32x4*>(v_s1 + o) = z;
    }
  }
  Entries E0, E1, EN;
  fetch(E0, 0);
  fetch(E1, 1);
  fetch(EN, 2);
  __syncthreads();  // the zeroing is done before any direct load lands
  uint32_t vb[NCH];  // bases of the next V load
  {
    uint32_t b0[NCH];
    bases(E0, 0, b0);
    dma(krs, klane, b0, k_s0);
    dma(vrs, vlane, b0, v_s0);
    put_bias(0, E0, 0);
  }
  if (T > 1) {
    bases(E1, 1, vb);
    dma(krs, klane, vb, k_s1);
    put_bias(1, E1, 1);
  }
  wait_dma_and_sync();
  f32x16 sA[2], sB[2];
  qk(k_s0, sA);
  {
    const float m_use = 0.f;
    float mt = logits(sA, 0, m_use);
    if (tail_s[0]) mt = mask_tail(sA, 0);
    rescale(sA, mt, m_use);
  }
  __syncthreads();  // every wave is done with k_s0 before K(2) overwrites it

  // EN holds the entries of tile n+2 (landed); vb the bases of V(n+1)
  auto iteration = [&](int n, auto PAR, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2]) {
    constexpr int p = decltype(PAR)::value;
    unsigned char* k_new = p ? k_s1 : k_s0;   // gets K(n+2)
    unsigned char* k_nxt = p ? k_s0 : k_s1;   // holds K(n+1)
    unsigned char* v_cur = p ? v_s1 : v_s0;   // holds V(n)
    unsigned char* v_new = p ? v_s0 : v_s1;   // gets V(n+1)
    uint32_t bn[NCH];
    if (n + 2 < T) {
      bases(EN, n + 2, bn);
      dma(krs, klane, bn, k_new);
      put_bias(p, EN, n + 2);
    }
    fetch(EN, n + 3);
    if (n + 1 < T) dma(vrs, vlane, vb, v_new);
    // phase A: QK(n+1) || probabilities of tile n
    qk(k_nxt, s_nxt);
    bf16x8 pf[4];
    l_run += probs(s_cur, pf);
    // phase B: PV(n) || logits of tile n+1
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    pv(v_cur, pf);
    float mt = logits(s_nxt, p ^ 1, m_use);
    if (n + 1 < T) {
      if (tail_s[p ^ 1]) mt = mask_tail(s_nxt, p ^ 1);
      rescale(s_nxt, mt, m_use);
    }
    wait_dma_and_sync();
#pragma unroll
    for (int j = 0; j < NCH; ++j) vb[j] = bn[j];
  };
#pragma unroll 1
  for (int n = 0; n < T; n += 2) {
    iteration(n, std::integral_constant<int, 0>{}, sA, sB);
    if (n + 1 < T) iteration(n + 1, std::integral_constant<int, 1>{}, sB, sA);
  }

  // ---- epilogue: O = O^T / l, valid queries only
  const float l_tot = half_swap_sum(l_run);
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
    case 64: return launch_t<D, BQ, 64, false>(a, st);
    default: return launch_t<D, BQ, 128, false>(a, st);
  }
}

// 128-query blocks run on the two-row kernel (absa_attend_pp.hip)
hipError_t launch_attend(const AttendLaunch& a, hipStream_t st, bool dense) {
  if (a.Bq == 128) return launch_attend_pp(a, st, dense);
  return a.d == 128 ? launch_bk<128, 64>(a, st, dense) : launch_bk<64, 64>(a, st, dense);
}

}  // namespace absa
