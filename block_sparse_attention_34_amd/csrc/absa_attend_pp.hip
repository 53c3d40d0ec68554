// Gather-attention for 128-query blocks on gfx950, two rows per workgroup in
// anti-phase (AB-Attention page, section "AB-Attention ve Üç Temel Yeniliği",
// third item: KV blocks much smaller than a tile are packed into full
// matrix-core tiles; SIP item: the 1/pi weights act inside the softmax
// numerator and denominator).  Dense attention is the same pipeline with
// contiguous KV tiles and unit weights.
//
// The arithmetic per tile is that of the one-row kernel (absa_attend.hip):
// S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 with the queries
// in the N position, so every lane owns one query and the softmax statistics
// stay in-lane.  What differs is the schedule.  A tile's work splits into a
// matrix phase (QK of the next tile and PV of the current one: 32 MFMAs and all
// LDS reads) and a vector phase (logits, running max, 2^t, bf16 rounding, row
// sums, and the direct loads of later tiles).  On a SIMD the matrix core and the
// vector ALU only overlap when the two streams come from different waves, so a
// workgroup holds two rows (8 waves, one wave of each row per SIMD) and runs
// them half a period apart: while row A's waves are in their matrix phase, row
// B's waves are in their vector phase, and the roles swap at every barrier.
//
// Before the phase loop each row loads tiles 0 and 1 and computes QK(0).  Then,
// per row, local phase j (row B runs one global step behind row A):
//   j = 2m        vector phase of tile m: softmax -> P(m); loads of K(m+2),
//                 V(m+1), bias(m+2) and the list entries of tile m+3
//   j = 2m + 1    matrix phase: QK(m+1) and PV(m)
// K and V have two LDS slots each, the bias four.  A load issued in the vector
// phase of tile m is first read two global steps later; each barrier waits only
// for the loads of earlier phases, so they stay in flight across one barrier.
#include <type_traits>

#include "absa_attend_tiles.h"
#include "absa_device.h"
#include "absa_launch.h"

namespace absa {

// ---- work queues of the persistent grid.  Queue x lists the row pairs the
// one-workgroup-per-pair grid deals to XCD x (its 32-pair slice of every full
// run of 256 pairs, then every eighth pair of the partial last run), in that
// order; a workgroup takes pairs from its own XCD's queue and, once that is
// empty, from the others in turn, so an XCD that runs slower (they do not all
// hold the same clock) hands its last pairs to the faster ones.
__global__ void queue_reset_kernel(int32_t* queue) {
  if (threadIdx.x < 8) queue[threadIdx.x] = 0;
}

// pair k of queue x, or -1 past its end
__device__ __forceinline__ int queue_pair(int x, int k, int npairs) {
  const int nfull = npairs / 256;
  if (k < 32 * nfull) return (k / 32) * 256 + x * 32 + (k % 32);
  const int p = nfull * 256 + (k - 32 * nfull) * 8 + x;
  return p < npairs ? p : -1;
}

// the next pair for this workgroup, or -1 when every queue is empty
__device__ __forceinline__ int take_pair(int32_t* queue, int npairs) {
  constexpr int kXccReg = (3 << 11) | 20;  // s_getreg_b32 operand: HW_REG_XCC_ID, bits [3:0]
  int x = (int)(__builtin_amdgcn_s_getreg(kXccReg) & 7u);
  for (int t = 0; t < 8; ++t) {
    const int p = queue_pair(x, atomicAdd(&queue[x], 1), npairs);
    if (p >= 0) return p;
    x = (x + 1) & 7;
  }
  return -1;
}

template <int D, int BK, bool DENSE, bool OUT_BF16, bool PC, bool PERSIST>
__global__ __launch_bounds__(512, 1) void attend_pp_kernel(AttendLaunch a) {
  constexpr int BQ = 128;
  constexpr int HT = 256;              // threads per row
  constexpr int NW = 4;                // waves per row, 32 queries each
  constexpr int CPR = D / 8;           // 16-byte chunks per key row
  constexpr int KPI = 64 / CPR;        // key rows covered by one wave-wide 16-byte load
  constexpr int NCH = 64 * CPR / HT;   // wave-wide loads per thread per tile and tensor
  constexpr int SPT = BK >= 64 ? 1 : 64 / BK;  // list entries per 64-key tile
  constexpr int TPE = BK > 64 ? BK / 64 : 1;   // 64-key tiles per list entry (128-key blocks: 2)
  constexpr int KS = D / 16;           // k-steps of the QK product
  constexpr int DB = D / 32;           // 32-wide d blocks of O
  constexpr int TILE = 64 * D * 2;
  constexpr float TAU = 8.f;           // the running max moves only when exceeded by this
  static_assert(BK % KPI == 0, "a wave-wide load must stay inside one block");
  static_assert(BK <= 64 || BK % 64 == 0, "a block larger than a tile spans whole tiles");
  static_assert(!(DENSE && BK != 64), "the dense path walks 64-key tiles");

  // Each K/V slot is an LDS object of its own and the phase loop is unrolled
  // by two, so every slot a phase touches is a compile-time constant: the
  // compiler can then tell that a phase's LDS reads never alias the direct
  // loads in flight into the other slots, and it adds no waits for them
  // (with one shared object it waited for every direct load before the
  // matrix phase's first V read).  [row][bytes]
  __shared__ __attribute__((aligned(16))) unsigned char k_s0[2][TILE], k_s1[2][TILE];
  __shared__ __attribute__((aligned(16))) unsigned char v_s0[2][TILE], v_s1[2][TILE];

  // Pairs of rows.  Workgroups are dealt round-robin over the 8 XCDs; within a
  // run of 8*32 workgroups, XCD x takes the 32 adjacent pairs [32x, 32x+32), i.e.
  // 64 adjacent query blocks of one head, whose lists overlap in that XCD's L2.
  // PERSIST: the grid is persistent: each workgroup takes pairs in the same XCD
  // order from the work queues until they are empty.  (A compile-time switch:
  // the one-pass instances then hold no loop state, which in this kernel's
  // scalar registers would spill.)
  const int npairs = (a.rows + 1) >> 1;
  __shared__ int next_pair;
  for (int pass = 0;; ++pass) {
  int pair;
  if constexpr (PERSIST) {
    if (threadIdx.x == 0) next_pair = take_pair(a.queue, npairs);
    __syncthreads();
    pair = next_pair;
    __syncthreads();  // (every wave has read it before the next take)
    if (pair < 0) break;
  } else {
    if (pass > 0) break;
    pair = blockIdx.x;
    constexpr int R = 32, S = 8 * R;
    const int g = pair / S, i = pair % S;
    if ((g + 1) * S <= npairs) pair = g * S + (i & 7) * R + (i >> 3);
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = wid >> 2, wq = wid & 3;
  const int h = lane >> 5, qn = lane & 31;
  unsigned char* const K0 = k_s0[half];
  unsigned char* const K1 = k_s1[half];
  unsigned char* const V0 = v_s0[half];
  unsigned char* const V1 = v_s1[half];

  auto list_len = [&](int r, int& nb) {
    if constexpr (DENSE) {
      nb = (a.L + BK - 1) / BK;
      return (a.L + 63) / 64;
    } else {
      int c = a.count[r];
      c = c < 0 ? 0 : (c > a.cap ? a.cap : c);
      nb = c;
      return TPE > 1 ? c * TPE : (c + SPT - 1) / SPT;
    }
  };
  const int row = 2 * pair + half, orow = 2 * pair + (1 - half);
  int nblk = 0, onb = 0;
  const int T = row < a.rows ? list_len(row, nblk) : 0;
  const int To = orow < a.rows ? list_len(orow, onb) : 0;
  const int rowc = row < a.rows ? row : a.rows - 1;  // a valid row for address arithmetic
  const int bh = rowc / a.NQ, qb = rowc % a.NQ;
  const size_t head_off = (size_t)bh * a.L * D;
  const int qi = qb * BQ + wq * 32 + qn;
  const bool qvalid = row < a.rows && qi < a.L;

  if (row < a.rows && T == 0 && qvalid) {  // empty list: the estimate is 0
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

  // ---- this lane's query, as the B operand of S^T = K Q^T
  bf16x8 qf[KS];
  {
    const u32x4* qp = reinterpret_cast<const u32x4*>(a.q + head_off + (size_t)(qvalid ? qi : 0) * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 w = qp[2 * ks + h];
      if (!qvalid) w = u32x4{0u, 0u, 0u, 0u};
      qf[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }
  const int32_t* lidx = DENSE ? nullptr : a.kv_idx + (size_t)rowc * a.cap;
  const float* lw = (DENSE || PC) ? nullptr : a.inv_pi + (size_t)rowc * a.cap;
  // Per-cluster lists: the row's list is the union of its clusters' samples;
  // lane l decodes entry l % SPT for cluster (l / SPT) % C, and each query takes
  // the bias of its own cluster (-inf where that cluster did not draw the block)
  const float* lwc = PC ? a.wc + (size_t)rowc * a.cap * a.C : nullptr;
  const int ccl = PC ? (lane / SPT) % a.C : 0;
  // (no labels: the row is two 64-query blocks, cluster j = block 2i + j of the pair)
  const int cq = PC ? (a.label ? (int)a.label[(size_t)rowc * BQ + wq * 32 + qn] : (wq >> 1)) : 0;

  // ---- direct loads (as in the one-row kernel): buffer resources cover this
  // head's K and V (L*D*2 bytes); rows past L lie past the end of the resource
  // and entries outside the list get a base past it, so such loads land zeros.
  const uint32_t head_bytes = (uint32_t)a.L * D * 2;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + head_off), 0, (int)head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.v + head_off), 0, (int)head_bytes, 0x00020000);
  constexpr uint32_t OOB = 0x7FFFFFF0u;
  uint32_t klane[NCH], vlane[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int kk = (j * NW + wq) * KPI + lane / CPR, cp = lane % CPR;
    klane[j] = (uint32_t)((kk % BK) * D * 2 + k_chunk<D>(kk, cp) * 16);
    vlane[j] = (uint32_t)((kk % BK) * D * 2 + v_chunk<D>(kk, cp) * 16);
  }
  // List entries, decoded lane-parallel: for a tile, lane i handles entry
  // tile*SPT + (i % SPT).  They are fetched one vector phase ahead with vector
  // loads, always (indices clamped to the list), so the destination registers
  // are reused in place.
  struct Entry {
    int blk;
    float w;
  };
  auto fetch = [&](Entry& E, int tile) {
    if constexpr (!DENSE) {
      const int last = nblk > 0 ? nblk - 1 : 0;
      const int e = TPE > 1 ? tile / TPE : tile * SPT + lane % SPT;
      const int ec = e < last ? e : last;
      E.blk = lidx[ec];
      E.w = PC ? lwc[(size_t)ec * a.C + ccl] : lw[ec];
    }
  };
  // A decoded tile: the wave-uniform byte base of each wave-wide load, the
  // bias log2(w) of each entry (lane i holds entry i; -inf for entries outside
  // the list), and the mask of its keys that lie past L (a listed block that
  // holds key L-1).
  struct Tile {
    float bias;
    unsigned long long past;
  };
  auto decode = [&](const Entry& E, int tile, uint32_t (&base)[NCH], Tile& t) {
    if constexpr (DENSE) {
#pragma unroll
      for (int j = 0; j < NCH; ++j) base[j] = (uint32_t)tile * (BK * D * 2);  // past the end: zeros
      t.bias = tile * 64 < a.L ? 0.f : -INFINITY;
      t.past = __ballot(tile * 64 < a.L && tile * 64 + lane >= a.L);
    } else {
      const int e = TPE > 1 ? tile / TPE : tile * SPT + lane % SPT;
      const bool ok = e < nblk && (unsigned)E.blk < (unsigned)a.NK;
      // (a block of several tiles: this tile's 64 keys start sub * 64 keys into it)
      const int sub = TPE > 1 ? tile % TPE : 0;
      const uint32_t bb = ok ? (uint32_t)E.blk * (BK * D * 2) + (uint32_t)sub * (64 * D * 2) : OOB;
#pragma unroll
      for (int j = 0; j < NCH; ++j)
        base[j] = __builtin_amdgcn_readlane(bb, TPE > 1 ? 0 : ((j * NW + wq) * KPI) / BK);
      t.bias = ok ? __log2f(E.w) : -INFINITY;
      t.past = 0ull;
      if constexpr (TPE > 1) {
        // one entry for the whole tile, key k at block row sub * 64 + k
        const int k0 = E.blk * BK + sub * 64;
        if (__ballot(ok && k0 + 64 > a.L) != 0ull) t.past = __ballot(ok && k0 + lane >= a.L);
      } else if (__ballot(ok && (E.blk + 1) * BK > a.L) != 0ull) {  // the block holding key L-1 (rare)
        // key k of the tile lies in entry k / BK, row k % BK
        int kb = 0;
        bool kok = false;
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
          const int bi = __builtin_amdgcn_readlane(E.blk, i);
          const bool oki = __builtin_amdgcn_readlane((int)ok, i) != 0;
          if (lane / BK == i) {
            kb = bi;
            kok = oki;
          }
        }
        t.past = __ballot(kok && kb * BK + lane % BK >= a.L);
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
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(buf + (j * NW + wq) * 1024), 16, off, 0, 0, 0);
    }
  };

  // ---- per-lane LDS read offsets
  int koff[KS];  // K rows qn (and qn + 32 at +32 rows), chunk 2 ks + h
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = k_off<D>(qn, 2 * ks + h);
  int voff[DB];  // V^T transposing reads: 16-lane group G, lane s in it
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
  f32x16 sacc[2];
  u32x4 pf[4];  // P of the current tile, bf16 pairs in the PV operand layout
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale_log2;
  bf16x2 ones;
  ones[0] = (__bf16)1.f;
  ones[1] = (__bf16)1.f;

  // ---- matrix work
  auto qk = [&](const unsigned char* kb) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[sb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const bf16x8 kfrag = *reinterpret_cast<const bf16x8*>(kb + koff[ks] + sb * 32 * (D * 2));
        sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag, qf[ks], sacc[sb], 0, 0, 0);
      }
  };
  auto pv = [&](const unsigned char* vb) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const unsigned char* p0 = vb + voff[db] + (16 * ks) * (D * 2);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + 8 * (D * 2)));
        const i16x4 w[2] = {lo, hi};
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w),
                                                          __builtin_bit_cast(bf16x8, pf[ks]), acc[db], 0, 0, 0);
      }
    }
  };

  // ---- vector work.  t = S scale log2(e) + log2(w) - m; a 4-key group of a
  // lane always lies in one entry, the same one for every lane; returns this
  // lane's max
  auto logits = [&](const Tile& tl, float m_use) {
    float cb[SPT];
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      if constexpr (PC)
        cb[i] = __shfl(tl.bias, SPT * cq + i, 64) - m_use;
      else
        cb[i] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tl.bias), i)) - m_use;
    }
    float mt = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const float cg = cb[(32 * sb + 8 * g4) / BK];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float tv = fmaf(sacc[sb][4 * g4 + i], sl2, cg);
          sacc[sb][4 * g4 + i] = tv;
          mt = fmaxf(mt, tv);
        }
      }
    return mt;
  };
  // a tile with keys past L: mask them individually and recompute the max
  // (element r of half sb holds key 32 sb + 8 (r / 4) + 4 h + r % 4)
  auto mask_tail = [&](const Tile& tl) {
    float mt = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const uint32_t w = (uint32_t)(tl.past >> (32 * sb)) >> (4 * h);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if ((w >> (8 * (r >> 2) + (r & 3))) & 1u) sacc[sb][r] = -INFINITY;
        mt = fmaxf(mt, sacc[sb][r]);
      }
    }
    return mt;
  };
  // move the reference when a tile exceeds it by more than TAU (or on the first
  // valid tile); afterwards sacc holds t relative to m_run
  // (The branch is taken by the whole wave when any lane needs it, lanes that
  // do not rescale by 1: a lane-divergent branch around the O^T accumulators
  // makes the compiler keep a second copy of them.)
  auto rescale = [&](float mt, float m_use) {
    mt = half_swap_max(mt);
    const bool need = mt > TAU || (m_run == -INFINITY && mt > -INFINITY);
    if (__ballot(need) != 0ull) {
      const float alpha = need ? ((m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(-mt)) : 1.f;
      const float shift = need ? mt : 0.f;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      m_run = need ? m_use + mt : m_run;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[sb][r] -= shift;
    }
  };

  // ---- the two rows' phase sequences on one barrier: row 0 runs vector(0),
  // matrix(0), vector(1), ... while row 1 runs the same sequence one step
  // later.  Both rows run the same number of iterations: phases of tiles past a row's
  // list are neutral (their K and V slots hold zeros, their bias is -inf, so P
  // is 0 and neither O, nor the running max, nor the row sum changes), which
  // keeps the loop free of branches around the accumulators.
  // Per-row pipeline state entering vector(m): sacc holds the logits of tile m
  // (relative to the reference in force when they were formed) and mt their
  // per-lane maximum; t1, t2 are the decoded tiles m+1, m+2 (vector(m) decodes
  // tile m+3 into t3); kn the K bases of tile m+2, vb the V bases of tile m+1;
  // EN the list entries of tile m+3.
  Entry EN;
  uint32_t kn[NCH], vb[NCH];
  Tile t1, t2, t3;
  float mt;
  auto form_logits = [&](const Tile& tl) {
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float x = logits(tl, m_use);
    if (tl.past != 0ull) x = mask_tail(tl);
    return x;
  };
  {
    Entry E0, E1, E2;
    fetch(E0, 0);
    fetch(E1, 1);
    fetch(E2, 2);
    fetch(EN, 3);
    uint32_t b0[NCH];
    Tile t0;
    decode(E0, 0, b0, t0);
    dma(krs, klane, b0, K0);
    dma(vrs, vlane, b0, V0);
    decode(E1, 1, vb, t1);
    dma(krs, klane, vb, K1);
    decode(E2, 2, kn, t2);
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    __syncthreads();
    qk(K0);
    mt = form_logits(t0);
  }

  // one direct load of a vector phase: chunk j of K(m+2) (j < NCH) or of
  // V(m+1) (j >= NCH), as dma() issues them
  auto dma_one = [&](int j, unsigned char* kbuf, unsigned char* vbuf) {
    const bool isk = j < NCH;
    const int jj = isk ? j : j - NCH;
    const int off = (int)((isk ? klane[jj] : vlane[jj]) + (isk ? kn[jj] : vb[jj]));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(isk ? krs : vrs, (lds_void_t*)((isk ? kbuf : vbuf) + (jj * NW + wq) * 1024),
                                             16, off, 0, 0, 0);
  };
  // P = 2^t of tile m rounded to bf16 in the PV operand layout (packed bf16
  // pairs: P lives across a barrier, and as a vector of single bf16 elements it
  // would occupy twice the registers); returns the row sum of exactly these
  // rounded values.  SPREAD: the phase's 2 NCH direct loads go out evenly
  // between the 16 pairs.  The four vector-phase waves of a CU share one
  // address unit; over gathered blocks, which often miss in L2, it then works
  // through the loads while the waves form P, where with the loads as one block
  // (which the compiler schedules ahead of the exponentials) each wave stalls
  // behind their queue.  The empty statements keep the pairs in this order
  // between the loads (the row sums stay free to move).  Over contiguous tiles
  // (dense), which hit in L2, the compiler's own placement of the block is
  // faster.
  auto probs_dma = [&](auto spread, unsigned char* kbuf, unsigned char* vbuf) {
    constexpr bool SPREAD = decltype(spread)::value;
    constexpr int EVERY = 16 / (2 * NCH);  // pairs per load
    float psum = 0.f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bf16x2 pk;
          pk[0] = (__bf16)__builtin_amdgcn_exp2f(sacc[sb][hf * 8 + 2 * e]);
          pk[1] = (__bf16)__builtin_amdgcn_exp2f(sacc[sb][hf * 8 + 2 * e + 1]);
          psum = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, psum, false);
          w[e] = __builtin_bit_cast(uint32_t, pk);
          if constexpr (SPREAD) {
            asm volatile("" ::"v"(w[e]));
            const int c = (sb * 2 + hf) * 4 + e;
            // load i after pair EVERY (i + 1), the last one after the final pair
            if ((c > 0 && c % EVERY == 0) || c == 15) {
              dma_one(c == 15 ? 2 * NCH - 1 : c / EVERY - 1, kbuf, vbuf);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
        pf[sb * 2 + hf] = w;
      }
    if constexpr (!SPREAD)
#pragma unroll
      for (int j = 0; j < 2 * NCH; ++j) dma_one(j, kbuf, vbuf);
    return psum;
  };
  // vector(m): softmax of tile m -> P(m), with the direct loads of K(m+2) and
  // V(m+1) spread between its pairs; then the decoding of tile m+3's entries
  // and the fetch of tile m+4's
  // (pc: the parity of m as a compile-time constant, which names the slots)
  auto vector_phase = [&](auto pc, int m) {
    constexpr int p = decltype(pc)::value;
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    rescale(mt, m_use);
    l_run += probs_dma(std::integral_constant<bool, !DENSE>(), p ? K1 : K0, p ? V0 : V1);  // K(m+2), V(m+1)
#pragma unroll
    for (int q = 0; q < NCH; ++q) vb[q] = kn[q];
    decode(EN, m + 3, kn, t3);
    fetch(EN, m + 4);
    // the loads of earlier phases have landed (this phase issued 2*NCH direct
    // loads after them, and loads return in order); this phase's may stay in
    // flight
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((2 * NCH) | 0x0070);  // vmcnt(2 NCH) lgkmcnt(0)
  };
  // matrix(m): QK(m+1) (past the list: zeros) and PV(m); then the logits of
  // tile m+1, which balances the two phases
  auto matrix_phase = [&](auto pc) {
    constexpr int p = decltype(pc)::value;
    qk(p ? K0 : K1);
    pv(p ? V1 : V0);
    // LDS reads run ahead of the matrix products that consume them: RA up
    // front, then one (K) or two (V) after every product
    constexpr int RA = 4;
    __builtin_amdgcn_sched_group_barrier(0x100, RA, 0);
#pragma unroll
    for (int i = 0; i < 2 * KS - RA / 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int i = 2 * KS - RA / 2; i < 2 * KS + 4 * DB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    mt = form_logits(t1);
    t1 = t2;
    t2 = t3;
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  };
  // barrier without a memory fence (each phase ends with its own waits); no
  // instruction may be scheduled across it, so the phases stay apart
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // Both rows run the same loop body; row 1 passes one barrier before it and
  // row 0 one after it, which puts row 1 one step behind (both execute
  // 2*NIT + 1 barriers, which the hardware counts per workgroup wherever they
  // sit in the code).
  const int NIT = T > To ? T : To;
  if (half == 1) barrier();
  const std::integral_constant<int, 0> even;
  const std::integral_constant<int, 1> odd;
#pragma unroll 1
  for (int it = 0; it < NIT; it += 2) {
    vector_phase(even, it);
    barrier();
    matrix_phase(even);
    barrier();
    if (it + 1 < NIT) {
      vector_phase(odd, it + 1);
      barrier();
      matrix_phase(odd);
      barrier();
    }
  }
  if (half == 0) barrier();

  // ---- epilogue: O = O^T / l, valid queries only
  if (T > 0) {
    const float l_tot = half_swap_sum(l_run);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    if (qvalid) {
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
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.o) + obase + dc) = make_float4(o0, o1, o2, o3);
          }
        }
    }
  }
  }  // next pair
}

template <int D, int BK, bool DENSE>
static hipError_t launch_pp_t(const AttendLaunch& a, hipStream_t st) {
  const int npairs = (a.rows + 1) / 2;
  if constexpr (!DENSE) {
    if (a.queue) {  // persistent grid over the work queues
      if (a.grid_limit < 1) return hipErrorInvalidValue;
      queue_reset_kernel<<<1, 64, 0, st>>>(a.queue);
      const dim3 grid(npairs < a.grid_limit ? npairs : a.grid_limit);
      if (a.wc) {
        if (a.out_bf16)
          attend_pp_kernel<D, BK, false, true, true, true><<<grid, 512, 0, st>>>(a);
        else
          attend_pp_kernel<D, BK, false, false, true, true><<<grid, 512, 0, st>>>(a);
      } else {
        if (a.out_bf16)
          attend_pp_kernel<D, BK, false, true, false, true><<<grid, 512, 0, st>>>(a);
        else
          attend_pp_kernel<D, BK, false, false, false, true><<<grid, 512, 0, st>>>(a);
      }
      return hipGetLastError();
    }
    if (a.wc) {
      if (a.out_bf16)
        attend_pp_kernel<D, BK, false, true, true, false><<<npairs, 512, 0, st>>>(a);
      else
        attend_pp_kernel<D, BK, false, false, true, false><<<npairs, 512, 0, st>>>(a);
      return hipGetLastError();
    }
  }
  if (a.queue) return hipErrorInvalidValue;
  if (a.out_bf16)
    attend_pp_kernel<D, BK, DENSE, true, false, false><<<npairs, 512, 0, st>>>(a);
  else
    attend_pp_kernel<D, BK, DENSE, false, false, false><<<npairs, 512, 0, st>>>(a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_pp_bk(const AttendLaunch& a, hipStream_t st, bool dense) {
  if (dense) return launch_pp_t<D, 64, true>(a, st);
  switch (a.Bk) {
    case 16: return launch_pp_t<D, 16, false>(a, st);
    case 32: return launch_pp_t<D, 32, false>(a, st);
    case 64: return launch_pp_t<D, 64, false>(a, st);
    default: return launch_pp_t<D, 128, false>(a, st);
  }
}

hipError_t launch_attend_pp(const AttendLaunch& a, hipStream_t st, bool dense) {
  return a.d == 128 ? launch_pp_bk<128>(a, st, dense) : launch_pp_bk<64>(a, st, dense);
}

}  // namespace absa
