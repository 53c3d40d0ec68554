// Block selection kernels for gfx950: KV block means, IBCS in-block k-means,
// IBCS block scoring and SIP sampling (AB-Attention page, section "AB-Attention
// ve Üç Temel Yeniliği", IBCS and SIP items).  The rules each kernel follows are
// listed in absa.h.  Everything is fp32 with correctly rounded divisions (the
// two contractions use split bf16 operands, exact for operands bf16 holds), so
// on inputs whose intermediates are exactly representable the lists and
// probabilities equal those of an exact computation.
#include "absa_attend_tiles.h"
#include "absa_device.h"
#include "absa_launch.h"

// No implicit multiply-add fusion: every product below is rounded on its own,
// as the selection arithmetic contract requires; fused steps are explicit fmaf.
#pragma clang fp contract(off)

namespace absa {

// 2^x on v_exp_f32.  On gfx950 it returns the exact power of two at every
// integer argument in [-126, 125] (checked on the device), and every argument
// used here is >= -64, so inputs whose logits are integers give exact terms.
__device__ __forceinline__ float exp2_split(float x) { return __builtin_amdgcn_exp2f(x); }

// ============================================================================= K1
// kbar^T[bh][c][b] = (1/n_b) sum_{valid keys of block b} K[bh][key][c] (written
// only when kbarT is not null), and the same means as bf16 head and tail, hi =
// bf16(kbar), lo = bf16(kbar - hi), the B operands of the logit product, in
// the matrix core's operand order: for each 32-block tile T and k-step s the
// 64 lanes' 16-byte operands lie contiguously, heads then tails,
// kbh[bh][T][s][hl][lane][8], lane (h, n) holding block 32 T + n, channels
// 16 s + 8 h .. + 7, so a wave reads each operand as one 1 KB piece.  Padding
// blocks (b >= NK) are 0.
// Grid (NKp/64, BH), 256 threads; a workgroup produces 64 blocks x D dims.
template <int D>
__global__ __launch_bounds__(256) void kv_block_mean_kernel(const uint16_t* __restrict__ k,
                                                            float* __restrict__ kbarT,
                                                            uint16_t* __restrict__ kbh, int L, int Bk,
                                                            int NK, int NKp) {
  constexpr int CPR = D / 8;            // 16-byte chunks per key row
  constexpr int BPP = 256 / CPR;        // blocks per pass
  constexpr int PASSES = 64 / BPP;
  __shared__ float tile[D][65];
  const int t = threadIdx.x;
  const int bh = blockIdx.y;
  const int b0 = blockIdx.x * 64;
  const uint16_t* kh = k + (size_t)bh * L * D;
  const int c = t % CPR;
#pragma unroll 1
  for (int p = 0; p < PASSES; ++p) {
    const int bl = p * BPP + t / CPR;
    const int b = b0 + bl;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    if (b < NK) {
      const int n = min(Bk, L - b * Bk);
      const uint4* src = reinterpret_cast<const uint4*>(kh + (size_t)b * Bk * D + c * 8);
#pragma unroll 1
      for (int r0 = 0; r0 < n; r0 += 16) {
        uint4 wv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)  // all loads in flight before the (ordered) sums
          wv[r] = (r0 + r < n) ? src[(size_t)(r0 + r) * (D / 8)] : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (r0 + r < n) {
            const uint4 w = wv[r];
            float lo, hi;
            unpack_bf16x2(w.x, lo, hi); acc[0] += lo; acc[1] += hi;
            unpack_bf16x2(w.y, lo, hi); acc[2] += lo; acc[3] += hi;
            unpack_bf16x2(w.z, lo, hi); acc[4] += lo; acc[5] += hi;
            unpack_bf16x2(w.w, lo, hi); acc[6] += lo; acc[7] += hi;
          }
        }
      }
      const float fn = (float)n;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = __fdiv_rn(acc[e], fn);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[c * 8 + e][bl] = acc[e];
  }
  __syncthreads();
  if (kbarT) {
    float* dst = kbarT + (size_t)bh * D * NKp + b0;
    for (int idx = t; idx < D * 64; idx += 256) {
      const int cc = idx >> 6, bl = idx & 63;
      dst[(size_t)cc * NKp + bl] = tile[cc][bl];
    }
  }
  // pieces (tile tt of the two here, k-step s, half hl, lane), 16 bytes each
  constexpr int KS = D / 16;
  for (int idx = t; idx < 2 * KS * 2 * 64; idx += 256) {
    const int ln = idx & 63, hl = (idx >> 6) & 1, ks = (idx >> 7) % KS, tt = (idx >> 7) / KS;
    const int bl = 32 * tt + (ln & 31), c0 = 16 * ks + 8 * (ln >> 5);
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = tile[c0 + e][bl];
      const __bf16 hi = (__bf16)x;
      v[e] = hl ? (__bf16)(x - (float)hi) : hi;
    }
    const size_t T = (size_t)bh * (NKp / 32) + (b0 / 32) + tt;
    *reinterpret_cast<bf16x8*>(kbh + (((T * KS + ks) * 2 + hl) * 64 + ln) * 8) = v;
  }
}

// ============================================================================= K2a
// Lloyd k-means of one query block (one workgroup per row).  Queries stay in
// token order; centroids start at members floor(j n / C); each step assigns
// every query to its nearest centroid (squared Euclidean, ties to the lowest
// j) and moves each non-empty centroid to the mean of its members.  Both
// contractions run on v_mfma_f32_32x32x16_bf16:
//  * assignment: G[j][q] = mu_j . x_q with the centroids split into bf16 high
//    and low parts (two products; exact for centroids representable in 16
//    significant bits, within 2^-17 relative otherwise); the nearest centroid
//    minimises |mu_j|^2 - 2 G[j][q] (|x|^2 is common to all j), ties to the
//    lowest j;
//  * update: sums[j][c] = sum_q [a(q) = j] x_q[c] as a product of a 0/1
//    assignment matrix with the query block (exact products, fp32 sums), then
//    one correctly rounded division by n_j.
template <int D>
__device__ __forceinline__ int xq_off(int q, int c) {  // byte offset of 16-byte chunk c of query row q
  if constexpr (D == 128) return q * 256 + ((c ^ (q & 15)) << 4);
  else return q * 128 + ((c ^ ((q >> 1) & 7)) << 4);
}

template <int D, int C>
__global__ __launch_bounds__(256) void ibcs_kmeans_mfma_kernel(const uint16_t* __restrict__ q,
                                                               float* __restrict__ mu_out,
                                                               int* __restrict__ nj_out,
                                                               uint8_t* __restrict__ lab_out, int L, int Bq,
                                                               int NQ, int Tk) {
  constexpr int KS = D / 16;   // k-steps of the assignment product
  constexpr int CH = D / 8;    // 16-byte chunks per row
  constexpr int NB = D / 32;   // 32-wide column blocks of the update product
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  __shared__ __attribute__((aligned(16))) unsigned char xs[128 * D * 2];
  __shared__ float mu_s[C][D];
  __shared__ __attribute__((aligned(16))) __bf16 mu_hi[C][D], mu_lo[C][D];
  __shared__ float musq[C];
  __shared__ __attribute__((aligned(16))) int lab[128];
  __shared__ int cnt[C];

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int h = lane >> 5, nn = lane & 31;
  const int row = blockIdx.x;
  const int bh = row / NQ, i = row % NQ;
  const int q0 = i * Bq;
  const int n = min(Bq, L - q0);

  // query block -> LDS (rows >= n are zero)
  {
    constexpr int PER = 128 * CH / 256;
    const u32x4* src = reinterpret_cast<const u32x4*>(q + ((size_t)bh * L + q0) * D);
    u32x4 wv[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int idx = t + 256 * j;
      wv[j] = (idx / CH < n) ? src[idx] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int idx = t + 256 * j;
      *reinterpret_cast<u32x4*>(xs + xq_off<D>(idx / CH, idx % CH)) = wv[j];
    }
  }
  __syncthreads();
  for (int idx = t; idx < C * D; idx += 256) {
    const int j = idx / D, c = idx % D;
    const int m = (j * n) / C;
    const uint16_t bits = *reinterpret_cast<const uint16_t*>(xs + xq_off<D>(m, c >> 3) + (c & 7) * 2);
    mu_s[j][c] = __uint_as_float((uint32_t)bits << 16);
  }
  __syncthreads();

#pragma unroll 1
  for (int step = 0; step < Tk; ++step) {
    // ---- split the centroids into bf16 parts, and |mu_j|^2
    for (int idx = t; idx < C * D; idx += 256) {
      const int j = idx / D, c = idx % D;
      const float m = mu_s[j][c];
      const __bf16 hi = (__bf16)m;
      mu_hi[j][c] = hi;
      mu_lo[j][c] = (__bf16)(m - (float)hi);
    }
    if (t < C) cnt[t] = 0;
    if (w < C) {  // wave w: |mu_w|^2 (fixed order: lane partial sums, then the wave sum)
      float sq = 0.f;
      for (int c = lane; c < D; c += 64) sq = fmaf(mu_s[w][c], mu_s[w][c], sq);
      sq = wave_sum(sq);
      if (lane == 0) musq[w] = sq;
    }
    if (C > 4 && w < C - 4) {
      float sq = 0.f;
      for (int c = lane; c < D; c += 64) sq = fmaf(mu_s[w + 4][c], mu_s[w + 4][c], sq);
      sq = wave_sum(sq);
      if (lane == 0) musq[w + 4] = sq;
    }
    __syncthreads();
    // ---- assignment: wave w owns queries 32 w .. 32 w + 31
    if (32 * w < n) {
      f32x16 g;
#pragma unroll
      for (int r = 0; r < 16; ++r) g[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 xb = *reinterpret_cast<const bf16x8*>(xs + xq_off<D>(32 * w + nn, 2 * ks + h));
        bf16x8 ah, al;
        if (nn < C) {
          ah = *reinterpret_cast<const bf16x8*>(&mu_hi[nn][16 * ks + 8 * h]);
          al = *reinterpret_cast<const bf16x8*>(&mu_lo[nn][16 * ks + 8 * h]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) { ah[e] = (__bf16)0.f; al[e] = (__bf16)0.f; }
        }
        g = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, xb, g, 0, 0, 0);
        g = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, xb, g, 0, 0, 0);
      }
      // lane (h, nn) register r holds centroid 8 (r/4) + 4 h + r%4 for query 32 w + nn
      float best = INFINITY;
      int bj = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 4 * h + r;
        if (j < C) {
          const float dj = musq[j] - 2.f * g[r];
          if (dj < best) { best = dj; bj = j; }
        }
      }
      if constexpr (C > 4) {
        const float ob = __shfl_xor(best, 32, 64);
        const int oj = __shfl_xor(bj, 32, 64);
        if (ob < best || (ob == best && oj < bj)) { best = ob; bj = oj; }
      }
      const int qq = 32 * w + nn;
      const bool valid = qq < n;
      if (h == 0) lab[qq] = valid ? bj : -1;
#pragma unroll
      for (int j = 0; j < C; ++j) {
        const unsigned long long m = __ballot(h == 0 && valid && bj == j);
        if (lane == 0 && m) atomicAdd(&cnt[j], (int)__popcll(m));
      }
    } else if (lane < 32) {
      lab[32 * w + lane] = -1;
    }
    __syncthreads();
    // ---- update: wave w owns columns 32 w .. 32 w + 31
    if (w < NB) {
      f32x16 sum;
#pragma unroll
      for (int r = 0; r < 16; ++r) sum[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {  // 16 queries per k-step
        // A: 0/1 assignment of queries 16 ks + {4h..4h+3, 8+4h..8+4h+3} to centroid nn
        const int4 la = *reinterpret_cast<const int4*>(&lab[16 * ks + 4 * h]);
        const int4 lb = *reinterpret_cast<const int4*>(&lab[16 * ks + 8 + 4 * h]);
        const int lv[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
        bf16x8 oh;
#pragma unroll
        for (int e = 0; e < 8; ++e) oh[e] = (__bf16)(lv[e] == nn ? 1.f : 0.f);
        // B: the same queries' values in columns 32 w + (lane & 31), read transposed
        const int G = lane >> 4, sl = lane & 15;
        const int col = 32 * w + 16 * (G & 1) + 4 * (sl & 3);
        const int qa = 16 * ks + 4 * h + (sl >> 2);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(xs + xq_off<D>(qa, col >> 3) + (col & 7) * 2));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(xs + xq_off<D>(qa + 8, col >> 3) + (col & 7) * 2));
        const i16x4 xv[2] = {lo, hi};
        sum = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oh, __builtin_bit_cast(bf16x8, xv), sum, 0, 0, 0);
      }
      // lane (h, nn) register r holds centroid 4 h + r (r < 4) for column 32 w + nn
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 4 * h + r;
        if (j < C && cnt[j] > 0) mu_s[j][32 * w + nn] = __fdiv_rn(sum[r], (float)cnt[j]);
      }
    }
    __syncthreads();
  }
  float* mo = mu_out + (size_t)row * C * D;
  for (int idx = t; idx < C * D; idx += 256) mo[idx] = mu_s[idx / D][idx % D];
  if (t < C) nj_out[(size_t)row * C + t] = cnt[t];
  // the last assignment of each query (per-cluster lists), 0 past the block's queries
  if (lab_out && t < Bq) lab_out[(size_t)row * Bq + t] = (uint8_t)(t < n ? lab[t] : 0);
}

// ============================================================================= K2b
// Block logits l[row][j][b] = alpha * (mu_j . kbar_b) for every centroid of a
// head against every KV block: a [NQ*C x d] x [d x NK] product on the bf16
// matrix core.  Each fp32 operand x is split into a bf16 head and tail,
// x = hi + lo + r with hi = bf16(x), lo = bf16(x - hi) and |r| <= 2^-17 |x|,
// and mu . kbar is formed as hi.hi' + hi.lo' + lo.hi' in one fp32 accumulator
// (per k-step, in that order): the dropped lo.lo' and remainder terms are
// below 2^-15 of each product, and operands that bf16 holds exactly (lo = 0)
// give the exact fp32 dot product.  The logits are formed twice and never
// stored: once for the normalisers, once for the scores.
// Workgroup = 4 waves x 32 centroids; a wave keeps its centroids' heads and
// tails as A operands in registers.  The means' heads and tails (split once,
// by K1, in operand order) pass through LDS one 32-block tile at a time, as a
// copy of the tile's bytes: every wave then reads its B operands as
// consecutive 16-byte pieces (no bank conflicts), and the global loads of a
// tile are issued two tiles ahead of its store into LDS.
// What a workgroup leaves depends on MODE:
//  * LG_MZ: per centroid, the running max m and normaliser
//    Z = sum nk 2^(l - m) over the split's blocks (terms more than 64 octaves
//    below the max dropped), combined over the lanes in a fixed order;
//  * LG_SCORE: with the max and normaliser of every centroid final (the
//    LG_MZ splits combined in split order), the mixture score of every row of
//    the wave's centroids and every block of the split,
//      s_b = sum_j (n_j/n) nk_b 2^(l_jb - m_j) / Z_j        (j in order),
//    into s[row][NKs];
//  * LG_SCORE_PC: per-cluster lists: each cluster's own score
//      s_jb = nk_b 2^(l_jb - m_j) / Z_j  into s[row C + j][NKs].
// Score rows have NKs = NK rounded up to 4 entries, the tail set to 0.
// Grid: ceil(M/128) x BH x nsplit workgroups in one dimension; split z covers a
// contiguous range of 32-block tiles.
constexpr int LG_MZ = 0, LG_SCORE = 1, LG_SCORE_PC = 2;

template <int D, int MODE, int C>
__global__ __launch_bounds__(256, 2) void ibcs_logit_kernel(const uint16_t* __restrict__ kbh,
                                                            const float* __restrict__ mu,
                                                            float2* __restrict__ mz,
                                                            const int* __restrict__ nj,
                                                            float* __restrict__ s_out, int M, int NK, int NKs,
                                                            int NKp, int L, int Bq, int Bk, int nsplit,
                                                            int tiles_per_split, float alpha) {
  constexpr int KS = D / 16;          // k-steps of 16 dims
  constexpr int TB = KS * 2048;       // bytes of one tile's operands (heads and tails)
  constexpr int NST = TB / (256 * 16);  // 16-byte pieces per thread and tile
  constexpr bool SCORE = MODE != LG_MZ;
  __shared__ __attribute__((aligned(16))) unsigned char kt[2][TB];
  __shared__ float mj_s[SCORE ? 128 : 1], coef_s[SCORE ? 128 : 1];
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform (scalar) index
  const int h = lane >> 5, n = lane & 31;
  // Workgroups are dealt to the 8 XCDs in turn; each XCD takes a contiguous
  // range of (centroid tile, head, split) triples, centroid tile fastest, so the
  // workgroups that read one head's split of the block means share an L2.
  const int ntm = (M + 127) / 128;
  const int G = (int)gridDim.x, g = (int)blockIdx.x, xcd = g & 7;
  const int nbh = G / (ntm * nsplit);
  const int u = xcd * (G >> 3) + min(xcd, G & 7) + (g >> 3);
  const int mt = u % ntm, bh = (u / ntm) % nbh, zs = u / (ntm * nbh);
  const int m0 = mt * 128 + w * 32;
  const int NT = NKp / 32;
  const int tile0 = zs * tiles_per_split;
  const int tile1 = min(NT, tile0 + tiles_per_split);
  const bool active = m0 < M;  // waves without centroids still stage tiles
  const unsigned char* kb = reinterpret_cast<const unsigned char*>(kbh) + (size_t)bh * NT * TB;

  if constexpr (SCORE) {
    // max, normaliser and score coefficient of the workgroup's 128 centroids:
    // (n_j/n)/Z_j for the mixture, 1/Z_j for a cluster's own score
    if (t < 128) {
      const int m = mt * 128 + t;
      float mx = -INFINITY, coef = 0.f;
      if (m < M) {
        const float2* pz = mz + ((size_t)bh * M + m) * nsplit;
        for (int z = 0; z < nsplit; ++z) mx = fmaxf(mx, pz[z].x);
        float zs = 0.f;
        for (int z = 0; z < nsplit; ++z) {
          const float d = pz[z].x - mx;
          if (d >= -64.f) zs = fmaf(pz[z].y, exp2_split(d), zs);
        }
        const int i = m / C;
        const int nq = min(Bq, L - i * Bq);
        const int cnt = nj[(size_t)bh * M + m];
        if (MODE == LG_SCORE) coef = (cnt > 0) ? __fdiv_rn(__fdiv_rn((float)cnt, (float)nq), zs) : 0.f;
        else coef = __fdiv_rn(1.f, zs);
      }
      mj_s[t] = mx;
      coef_s[t] = coef;
    }
  }

  // A operands: lane (h, n) holds mu[m0 + n][16 s + 8 h + e], e = 0..7, as head and tail
  bf16x8 ahi[KS], alo[KS];
  {
    const int m = m0 + n;
    const f32x4* src = reinterpret_cast<const f32x4*>(mu + ((size_t)bh * M + (m < M ? m : 0)) * D);
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
      for (int q4 = 0; q4 < 2; ++q4) {
        f32x4 x4 = src[4 * s2 + 2 * h + q4];
        if (m >= M) x4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const __bf16 hi = (__bf16)x4[e];
          ahi[s2][4 * q4 + e] = hi;
          alo[s2][4 * q4 + e] = (__bf16)(x4[e] - (float)hi);
        }
      }
  }
  auto fetch = [&](u32x4 (&stage)[NST], int tile) {
#pragma unroll
    for (int i = 0; i < NST; ++i)
      stage[i] = *reinterpret_cast<const u32x4*>(kb + (size_t)tile * TB + (t + 256 * i) * 16);
  };
  auto put = [&](const u32x4 (&stage)[NST], int buf) {
#pragma unroll
    for (int i = 0; i < NST; ++i) *reinterpret_cast<u32x4*>(&kt[buf][(t + 256 * i) * 16]) = stage[i];
  };
  u32x4 stA[NST], stB[NST];
  fetch(stA, tile0);
  put(stA, 0);
  if (tile0 + 1 < tile1) fetch(stA, tile0 + 1);

  const int rows_here = max(0, min(32, M - m0));  // the wave's centroids below M
  float rm[16], rz[16];  // LG_MZ: running max and normaliser of the lane's 16 centroids
  float mj[16], cf[16];  // scores: final max and coefficient of the lane's 16 centroids
#pragma unroll
  for (int r = 0; r < 16; ++r) { rm[r] = -INFINITY; rz[r] = 0.f; mj[r] = 0.f; cf[r] = 0.f; }
  if constexpr (SCORE) {
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = w * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      mj[r] = mj_s[m];
      cf[r] = coef_s[m];
    }
  }
  // LG_SCORE: first score row of the wave's centroids (rows m0/C ..); LG_SCORE_PC: row of centroid m0
  float* const srow = (MODE == LG_SCORE) ? s_out + ((size_t)bh * (M / C) + m0 / C) * NKs
                                         : s_out + ((size_t)bh * M + m0) * NKs;
  const int nrows_w = (MODE == LG_SCORE) ? rows_here / C : rows_here;

  // Score stores go through a buffer resource over the wave's score rows
  // (nrows_w rows of NKs entries): rows past them fall outside it, and a lane
  // with nothing to store aims at an offset past its end; such stores are
  // dropped, so the epilogue below is straight-line code.
  constexpr uint32_t OOB = 0x7FFFFFF0u;
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(SCORE && active ? srow : s_out), 0, SCORE && active ? nrows_w * NKs * 4 : 0, 0x00020000);
  // The logits of one tile (its B operands from LDS buffer buf)
  auto logits = [&](int buf) {
    const unsigned char* kl = &kt[buf][lane * 16];
    bf16x8 bhi[KS], blo[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bhi[ks] = *reinterpret_cast<const bf16x8*>(kl + ks * 2048);
      blo[ks] = *reinterpret_cast<const bf16x8*>(kl + ks * 2048 + 1024);
    }
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[ks], bhi[ks], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[ks], blo[ks], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo[ks], bhi[ks], acc, 0, 0, 0);
    }
    return acc;
  };
  // What a tile's logits leave (tile0 - 1 stands for "no tile yet": every block is padding)
  auto epilogue = [&](const f32x16& acc, int tile) {
    const int b = tile * 32 + n;
    const bool started = tile >= tile0;
    const bool bv = started && b < NK;
    const float nk = (float)min(Bk, L - b * Bk);
    if constexpr (SCORE) {
      // lane (h, n) register r: centroid m0 + 8 (r/4) + 4 h + r%4 against block b
      const bool bs = started && b < NKs;  // the row's entry b exists (zero past NK)
      float term[16];
      uint32_t ok = 0u;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float dl = fmaf(alpha, acc[r], -mj[r]);
        const bool on = dl >= -64.f && cf[r] != 0.f;
        term[r] = on ? nk * exp2_split(dl) : 0.f;
        ok |= on ? (1u << r) : 0u;
      }
      auto put_score = [&](int rl, float sv, bool lane_stores) {
        const uint32_t off = (bs && lane_stores) ? (uint32_t)(rl * NKs + b) * 4u : OOB;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(bv ? sv : 0.f), srs, off, 0, 0);
      };
      if constexpr (MODE == LG_SCORE_PC) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          put_score(8 * (r >> 2) + 4 * h + (r & 3), ((ok >> r) & 1u) ? fmaf(cf[r], term[r], 0.f) : 0.f, true);
      } else if constexpr (C <= 4) {
        // the C centroids of a row are consecutive registers of one lane
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int gg = 0; gg < 4 / C; ++gg) {
            float sv = 0.f;
#pragma unroll
            for (int j = 0; j < C; ++j) {
              const int r = 4 * q + gg * C + j;
              sv = ((ok >> r) & 1u) ? fmaf(cf[r], term[r], sv) : sv;
            }
            put_score((8 * q + 4 * h + gg * C) / C, sv, true);
          }
      } else {
        // C = 8: row q's centroids 0..3 sit in half-wave 0 (registers 4 q ..),
        // 4..7 in half-wave 1; half 1 continues the sum half 0 started
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float sv = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            sv = (h == 0 && ((ok >> (4 * q + j)) & 1u)) ? fmaf(cf[4 * q + j], term[4 * q + j], sv) : sv;
          sv = __shfl_xor(sv, 32, 64);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            sv = ((ok >> (4 * q + j)) & 1u) ? fmaf(cf[4 * q + j], term[4 * q + j], sv) : sv;
          put_score(q, sv, h == 1);
        }
      }
    } else {
      // Online (m, Z): with d = |m - l| only one of the two factors 2^(m - max)
      // and 2^(l - max) differs from 1, so one exp2 per logit suffices: a new
      // max gives Z e + nk, an old one Z + nk e.  Padding blocks (b >= NK)
      // enter as l = -inf, which changes neither m nor Z; fma(alpha, acc, 0)
      // rounds like the product alone.
      const float pad = bv ? 0.f : -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float l = fmaf(alpha, acc[r], pad);
        const float dd = fabsf(rm[r] - l);
        const float e = dd <= 64.f ? exp2_split(-dd) : 0.f;
        const bool up = l > rm[r];
        rz[r] = up ? fmaf(rz[r], e, nk) : fmaf(nk, e, rz[r]);
        rm[r] = fmaxf(rm[r], l);
      }
    }
  };
  // Software pipeline by one tile: the matrix core works on tile t while the
  // vector units finish tile t - 1, in the same stretch of straight-line code.
  f32x16 accp;
#pragma unroll
  for (int r = 0; r < 16; ++r) accp[r] = 0.f;
  auto body = [&](int tile, const u32x4 (&sput)[NST], u32x4 (&sfetch)[NST]) {
    const int buf = (tile - tile0) & 1;
    __syncthreads();
    if (tile + 2 < tile1) fetch(sfetch, tile + 2);
    if (active) {
      const f32x16 accn = logits(buf);
      epilogue(accp, tile - 1);
      accp = accn;
      // interleave: the tile's operand reads first, then each product with a share of the epilogue
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * KS, 0);
#pragma unroll
      for (int i = 0; i < 3 * KS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
      }
    }
    if (tile + 1 < tile1) put(sput, buf ^ 1);
  };
#pragma unroll 1
  for (int tile = tile0; tile < tile1; tile += 2) {
    body(tile, stA, stB);
    if (tile + 1 < tile1) body(tile + 1, stB, stA);
  }
  if (active) epilogue(accp, tile1 - 1);
  if constexpr (!SCORE) {
    if (!active) return;
    // combine over the 32 blocks (lanes) of each half-wave and write this split's
    // partial (m, Z) of every centroid
#pragma unroll
    for (int r = 0; r < 16; ++r) {
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) {
        const float m2 = __shfl_xor(rm[r], o, 64), z2 = __shfl_xor(rz[r], o, 64);
        const float mn = fmaxf(rm[r], m2);
        const float d0 = rm[r] - mn, d1 = m2 - mn;
        const float e0 = d0 >= -64.f ? exp2_split(d0) : 0.f;
        const float e1 = d1 >= -64.f ? exp2_split(d1) : 0.f;
        rz[r] = fmaf(rz[r], e0, z2 * e1);
        rm[r] = mn;
      }
      const int m = m0 + 8 * (r >> 2) + 4 * h + (r & 3);
      if (n == 0 && m < M) mz[((size_t)bh * M + m) * nsplit + zs] = make_float2(rm[r], rz[r]);
    }
  }
}

// ============================================================================= K3
// Sampling: the row's list (one list per row) or the list of cluster j of a
// row (per-cluster lists: list row C + j, the full budget, Philox counter word
// i C + j; a cluster without members gets an empty list), held by WPL waves
// (one for NK <= 5120, two up to 8192, four beyond).  The list's blocks are
// laid out over 256 WPL layout threads of P contiguous blocks each (P a
// multiple of 4, the smallest with 256 WPL P >= NK, and exactly the kernel's
// compile-time chunk size); lane l of wave w holds the chunks of layout
// threads 256 w + 64 v + l, v = 0..3, in registers for the whole list:
//  * SIP capping rounds in straight-line code.  A block is free while its
//    register holds a positive score; capping sets it to -0, which adds
//    nothing to a sum, is never capped again and stays apart from a zero
//    score.  Every sum is taken in the layout's thread order (per-thread
//    partials in block order, wave totals, the four wave totals in order);
//  * top-k: the threshold bit pattern by bisection on the same registers,
//    then the lowest-index ties;
//  * the decisions: probability (1 capped, s R / S_U other positive scores, 0
//    else), one Philox block per 4 consecutive blocks, and the list entries
//    in block order (thread-order prefix sums).
// With one wave per list there is no LDS and no barrier (four lists per
// workgroup).  With several, the workgroup is the list and every total and
// prefix crosses the waves through LDS after a barrier; all of the list's
// waves see the same totals, so they take the same branches and barriers.
constexpr int SR_WAVES = 4;  // lists per workgroup with one wave per list

__device__ __forceinline__ bool is_neg_zero(float x) { return __float_as_uint(x) == 0x80000000u; }

constexpr int SR_SIP = 0, SR_TOPK = 1;

// (at least three waves per SIMD: the kernel is bound by its vector work and
// latency, and the 20-block chunks fit in the 168 registers that allows)
template <int PM, int MODE, int WPL>
__global__ __launch_bounds__(64 * (WPL == 1 ? SR_WAVES : WPL), 3) void sip_rows_kernel(SelectLaunch a, int nlists,
                                                                                     int NKs) {
  static_assert(PM % 4 == 0 && (WPL == 1 || WPL == 2 || WPL == 4), "chunk size and waves per list");
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lst = WPL == 1 ? blockIdx.x * SR_WAVES + wv : blockIdx.x;
  const int wl = WPL == 1 ? 0 : wv;  // this wave's part of the list
  if (lst >= nlists) return;         // (uniform over a list's waves)
  const int C = a.C;
  const int row = a.per_cluster ? lst / C : lst;
  const int jc = a.per_cluster ? lst - row * C : 0;
  const int bh = row / a.NQ, i = row - bh * a.NQ;
  const int NK = a.NK;
  if (a.per_cluster && a.nj[(size_t)row * C + jc] == 0) {
    if (lane == 0 && wl == 0) a.count[lst] = 0;
    return;
  }
  const uint32_t ctr1 = a.per_cluster ? (uint32_t)(i * C + jc) : (uint32_t)i;
  // blocks per layout thread: equal to PM (the launch picks the instance), but
  // formed at run time, which keeps the chunk addressing as cheap in registers
  const int P = 4 * ((NK + 1024 * WPL - 1) / (1024 * WPL));
  // The layout threads' chunks in registers.  The row holds NKs entries (a
  // multiple of 4, zero past NK) behind a buffer resource of that size: every
  // 16-byte piece lies wholly inside or wholly past its end, and the pieces
  // past it read as 0, so chunk padding is 0 without a per-element test (and
  // lies after every block: the chunks tile [0, 256 WPL P) exactly).
  const __amdgpu_buffer_rsrc_t srs =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(a.s + (size_t)lst * NKs), 0, NKs * 4, 0x00020000);
  int b0[4];
  float sv[4][PM];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int bt = (64 * (4 * wl + v) + lane) * P;
    b0[v] = bt;
#pragma unroll
    for (int e = 0; e < PM; e += 4) {
      const u32x4 x4 = __builtin_amdgcn_raw_buffer_load_b128(srs, (bt + e) * 4, 0, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q) sv[v][e + q] = __uint_as_float(x4[q]);
    }
  }
  // Sums over the list's waves in wave order, through one of two LDS slots
  // (alternating, so a wave that runs ahead to the next exchange cannot
  // overwrite a slot another wave still reads: it must pass the barrier of
  // the exchange in between first).
  __shared__ float xf[2][WPL];
  __shared__ int xi[2][WPL];
  int xk = 0;
  auto across = [&](float t) {
    if constexpr (WPL == 1) {
      return t;
    } else {
      if (lane == 0) xf[xk][wl] = t;
      __syncthreads();
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < WPL; ++w) s += xf[xk][w];
      xk ^= 1;
      return s;
    }
  };
  // (the int exchange also returns the sum of the waves before this one)
  auto across_i = [&](int t, int& before) {
    before = 0;
    if constexpr (WPL == 1) {
      return t;
    } else {
      if (lane == 0) xi[xk][wl] = t;
      __syncthreads();
      int s = 0;
#pragma unroll
      for (int w = 0; w < WPL; ++w) {
        const int x = xi[xk][w];
        before += w < wl ? x : 0;
        s += x;
      }
      xk ^= 1;
      return s;
    }
  };
  // totals in the layout's thread order
  auto total4 = [&](const float (&x)[4]) {
    float t = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) t += wave_total(x[v]);
    return across(t);
  };
  auto total4i = [&](const int (&x)[4]) {
    int t = 0, before;
#pragma unroll
    for (int v = 0; v < 4; ++v) t += wave_total_i(x[v]);
    return across_i(t, before);
  };
  // exclusive prefix of per-thread counts in the layout's thread order, and the total
  auto scan4 = [&](const int (&x)[4], int (&off)[4]) {
    int base = 0, before;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int inc = wave_inclusive_scan(x[v], lane);
      off[v] = base + inc - x[v];
      base += __shfl(inc, 63, 64);
    }
    const int total = across_i(base, before);
#pragma unroll
    for (int v = 0; v < 4; ++v) off[v] += before;
    return total;
  };

  uint64_t km[4] = {0ull, 0ull, 0ull, 0ull};  // kept blocks of each chunk
  if constexpr (MODE == SR_SIP) {
    float Rb = a.nstar, S_U;
    float part[4];
    int cnt[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      part[v] = 0.f;
      cnt[v] = 0;
#pragma unroll
      for (int e = 0; e < PM; ++e) {
        part[v] += sv[v][e];
        cnt[v] += sv[v][e] > 0.f;
      }
    }
    S_U = total4(part);
    int nfree = total4i(cnt);
#pragma unroll 1
    while (nfree > 0) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        part[v] = 0.f;
        cnt[v] = 0;
#pragma unroll
        for (int e = 0; e < PM; ++e) {
          const float x = sv[v][e];
          const bool cp = __fmul_rn(x, Rb) >= S_U;  // never for 0 or -0: S_U > 0 while blocks are free
          cnt[v] += cp;
          sv[v][e] = cp ? -0.f : x;
          part[v] += sv[v][e];
        }
      }
      const float tp = total4(part);
      const int tc = total4i(cnt);
      if (tc == 0) break;
      S_U = tp;
      Rb -= (float)tc;
      nfree -= tc;
    }
    // probabilities (kept in sv) and draws; chunk padding has probability 0
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int g = 0; g < PM; g += 4) {
        const philox_u4 x = philox4x32_10({(uint32_t)((b0[v] + g) >> 2), ctr1, (uint32_t)bh, a.ctr3}, a.key0, a.key1);
        const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int e = g + q;
          const float sc = sv[v][e];
          const float pr = is_neg_zero(sc) ? 1.f : (sc > 0.f) ? __fdiv_rn(__fmul_rn(sc, Rb), S_U) : 0.f;
          km[v] |= ((float)(xw[q] >> 8) * 0x1p-24f < pr) ? (1ull << e) : 0ull;
          sv[v][e] = pr;
        }
        // one group at a time: interleaving the unrolled generators would only cost registers
        __builtin_amdgcn_sched_barrier(0);
      }
  } else {
    // the largest bit pattern with #{s >= pattern} >= k* (chunk padding is 0, never counted)
    uint32_t lo = 0u, hi = 0x7F800001u;
#pragma unroll 1
    while (hi - lo > 1u) {
      const uint32_t mid = lo + ((hi - lo) >> 1);
      int c = 0;
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int e = 0; e < PM; ++e) c += (__float_as_uint(sv[v][e]) >= mid);
      int before;
      if (across_i(wave_total_i(c), before) >= a.kstar) lo = mid; else hi = mid;
    }
    int gt[4], eq[4], rank[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      gt[v] = 0;
      eq[v] = 0;
#pragma unroll
      for (int e = 0; e < PM; ++e) {
        const uint32_t u = __float_as_uint(sv[v][e]);
        gt[v] += (u > lo);
        eq[v] += (u == lo);
      }
    }
    // (chunk padding is 0 and comes after every block in thread order: when the
    // threshold is 0, the ties kept, the lowest-index ones, are all real blocks)
    const int need = a.kstar - total4i(gt);
    scan4(eq, rank);
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int e = 0; e < PM; ++e) {
        const uint32_t u = __float_as_uint(sv[v][e]);
        bool keep = u > lo;
        if (u == lo) keep = rank[v]++ < need;
        km[v] |= keep ? (1ull << e) : 0ull;
        sv[v][e] = keep ? 1.f : 0.f;
      }
  }
  // list entries in block order
  int nk4[4], off[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) nk4[v] = __popcll(km[v]);
  const int total = scan4(nk4, off);
  int32_t* idx_row = a.kv_idx + (size_t)lst * a.cap;
  float* w_row = a.inv_pi + (size_t)lst * a.cap;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    int o = off[v];
#pragma unroll
    for (int e = 0; e < PM; ++e)
      if ((km[v] >> e) & 1ull) {
        idx_row[o] = b0[v] + e;
        w_row[o] = MODE == SR_SIP ? __frcp_rn(sv[v][e]) : 1.f;
        ++o;
      }
  }
  if (a.pi_out) {  // inspection (one list per row): stores past NK fall outside the resource
    const __amdgpu_buffer_rsrc_t prs =
        __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(a.pi_out + (size_t)lst * NK), 0, NK * 4, 0x00020000);
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int e = 0; e < PM; ++e)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sv[v][e]), prs, (b0[v] + e) * 4, 0, 0);
  }
  if (lane == 0 && wl == 0) a.count[lst] = total;
}

// Lists that keep every block with probability 1 (SIP with n* >= NK, top-k
// with k* >= NK, ALL), or none (top-k with k* = 0): one list per workgroup.
__global__ __launch_bounds__(256) void sel_all_kernel(SelectLaunch a, int keep_all) {
  const int lst = blockIdx.x;
  const int C = a.C;
  const int row = a.per_cluster ? lst / C : lst;
  const int jc = a.per_cluster ? lst - row * C : 0;
  const bool empty = !keep_all || (a.per_cluster && a.nj[(size_t)row * C + jc] == 0);
  const int NK = a.NK;
  if (!empty) {
    for (int b = threadIdx.x; b < NK; b += 256) {
      a.kv_idx[(size_t)lst * a.cap + b] = b;
      a.inv_pi[(size_t)lst * a.cap + b] = 1.f;
    }
  }
  if (a.pi_out)
    for (int b = threadIdx.x; b < NK; b += 256) a.pi_out[(size_t)lst * NK + b] = keep_all ? 1.f : 0.f;
  if (threadIdx.x == 0) a.count[lst] = empty ? 0 : NK;
}

// ============================================================================= per-cluster union
constexpr int SIP_NT = 256;

// One workgroup per row: the ascending union of the row's C cluster lists and
// the weight of every (entry, cluster) pair, 0 where the cluster did not draw
// the block.  LDS holds one word per KV block: the cluster mask in the low 8
// bits, the union position above it.  The weight rows are zeroed with
// contiguous stores, then each cluster's drawn weights are scattered in.
// With NQi > 0 the same union is taken over pairs of 64-query rows (C = 2):
// output row bh NQo + i joins the lists of rows bh NQi + 2i and bh NQi + 2i + 1
// (the second absent when 2i + 1 = NQi).
__global__ __launch_bounds__(SIP_NT) void cluster_union_kernel(const int32_t* __restrict__ ccount,
                                                               const int32_t* __restrict__ cidx,
                                                               const float* __restrict__ cw, int ccap, int C,
                                                               int NK, int32_t* __restrict__ ucount,
                                                               int32_t* __restrict__ uidx, float* __restrict__ uw,
                                                               int ucap, int NQo, int NQi) {
  extern __shared__ uint32_t slot[];  // [NK]
  __shared__ int redi[2 * (SIP_NT / 64)];
  const int t = threadIdx.x;
  const size_t row = blockIdx.x;
  // list j of this row: row C + j, or (NQi > 0: pairs of 64-query blocks) block 2i + j
  // of head bh for row bh NQo + i, absent past the head's last block
  auto list_of = [&](int j, int& n) -> size_t {
    size_t li = row * C + j;
    bool ok = true;
    if (NQi > 0) {
      const size_t bh = row / NQo, i = row % NQo;
      ok = 2 * i + j < (size_t)NQi;
      li = bh * NQi + 2 * i + j;
    }
    n = ok ? min(ccount[li], ccap) : 0;
    return li;
  };
  for (int b = t; b < NK; b += SIP_NT) slot[b] = 0u;
  __syncthreads();
  for (int j = 0; j < C; ++j) {
    int n;
    const int32_t* li = cidx + list_of(j, n) * ccap;
    for (int e = t; e < n; e += SIP_NT) {
      const int b = li[e];
      if ((unsigned)b < (unsigned)NK) atomicOr(&slot[b], 1u << j);
    }
  }
  __syncthreads();
  const int P = (NK + SIP_NT - 1) / SIP_NT;  // contiguous chunk of blocks per thread
  const int b0 = min(NK, t * P), b1 = min(NK, b0 + P);
  int mine = 0;
  for (int b = b0; b < b1; ++b) mine += slot[b] != 0u;
  int total;
  int pos = block_exclusive_scan<SIP_NT>(mine, redi, total);
  float* wrow = uw + row * ucap * C;
  for (int b = b0; b < b1; ++b) {
    const uint32_t m = slot[b];
    if (m) {
      uidx[row * ucap + pos] = b;
      slot[b] = ((uint32_t)pos << 8) | m;
      ++pos;
    }
  }
  // every weight of the union starts at 0 (coalesced); the drawn ones follow
  // after the barrier, which also orders these stores before them
  for (int i = t; i < total * C; i += SIP_NT) wrow[i] = 0.f;
  __syncthreads();
  for (int j = 0; j < C; ++j) {
    int n;
    const size_t lr = list_of(j, n);
    const int32_t* li = cidx + lr * ccap;
    const float* lw = cw + lr * ccap;
    for (int e = t; e < n; e += SIP_NT) {
      const int b = li[e];
      if ((unsigned)b < (unsigned)NK) wrow[(size_t)(slot[b] >> 8) * C + j] = lw[e];
    }
  }
  if (t == 0) ucount[row] = total;
}

hipError_t launch_pair_union(const PairUnionLaunch& a, hipStream_t st) {
  cluster_union_kernel<<<a.rows_out, SIP_NT, (size_t)a.NK * sizeof(uint32_t), st>>>(
      a.count, a.kv_idx, a.inv_pi, a.cap, 2, a.NK, a.ucount, a.uidx, a.uw, a.ucap, a.NQo, a.NQi);
  return hipGetLastError();
}

// ============================================================================= launchers
template <int D>
static void launch_logit(const SelectLaunch& a, int mode, dim3 grid, hipStream_t st, int M, int NKs, int nsplit,
                         int per) {
#define ABSA_LG(MM, CC)                                                                                     \
  ibcs_logit_kernel<D, MM, CC><<<grid, 256, 0, st>>>(a.kbh, a.mu, a.mz, a.nj, a.s, M, a.NK, NKs, a.NKp, a.L, a.Bq, \
                                                     a.Bk, nsplit, per, a.alpha)
  if (mode == LG_MZ) {
    ABSA_LG(LG_MZ, 1);
  } else if (mode == LG_SCORE_PC) {
    ABSA_LG(LG_SCORE_PC, 1);
  } else {
    switch (a.C) {
      case 1: ABSA_LG(LG_SCORE, 1); break;
      case 2: ABSA_LG(LG_SCORE, 2); break;
      case 4: ABSA_LG(LG_SCORE, 4); break;
      default: ABSA_LG(LG_SCORE, 8); break;
    }
  }
#undef ABSA_LG
}

hipError_t launch_select(const SelectLaunch& a, hipStream_t st, hipEvent_t* ev) {
  int nev = 0;
  auto mark = [&]() -> hipError_t { return ev ? hipEventRecord(ev[nev++], st) : hipSuccess; };
  const int BH = a.B * a.H;
  const int rows = BH * a.NQ;
  const int NKs = (a.NK + 3) & ~3;
  {
    hipError_t e = mark();
    if (e != hipSuccess) return e;
  }
  // K1
  {
    dim3 grid(a.NKp / 64, BH);
    if (a.d == 128)
      kv_block_mean_kernel<128><<<grid, 256, 0, st>>>(a.k, a.kbarT, a.kbh, a.L, a.Bk, a.NK, a.NKp);
    else
      kv_block_mean_kernel<64><<<grid, 256, 0, st>>>(a.k, a.kbarT, a.kbh, a.L, a.Bk, a.NK, a.NKp);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = mark();
    if (e != hipSuccess) return e;
  }
  // K2a
  {
#define ABSA_KM(DD, CC) \
  ibcs_kmeans_mfma_kernel<DD, CC><<<rows, 256, 0, st>>>(a.q, a.mu, a.nj, a.label, a.L, a.Bq, a.NQ, a.Tk)
    if (a.d == 128) {
      switch (a.C) {
        case 1: ABSA_KM(128, 1); break;
        case 2: ABSA_KM(128, 2); break;
        case 4: ABSA_KM(128, 4); break;
        default: ABSA_KM(128, 8); break;
      }
    } else {
      switch (a.C) {
        case 1: ABSA_KM(64, 1); break;
        case 2: ABSA_KM(64, 2); break;
        case 4: ABSA_KM(64, 4); break;
        default: ABSA_KM(64, 8); break;
      }
    }
#undef ABSA_KM
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = mark();
    if (e != hipSuccess) return e;
  }
  // K2b: per-split (max, normaliser) of every centroid, then the scores
  int per;
  const int nsplit = logit_splits(a.NQ, a.C, BH, a.NKp, &per);
  const int M = a.NQ * a.C;
  const dim3 lgrid(((M + 127) / 128) * BH * nsplit);
  for (int pass = 0; pass < 2; ++pass) {
    const int mode = pass == 0 ? LG_MZ : (a.per_cluster ? LG_SCORE_PC : LG_SCORE);
    if (a.d == 128) launch_logit<128>(a, mode, lgrid, st, M, NKs, nsplit, per);
    else launch_logit<64>(a, mode, lgrid, st, M, NKs, nsplit, per);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = mark();
    if (e != hipSuccess) return e;
  }
  // K3: one list per wave
  {
    const int nlists = a.per_cluster ? rows * a.C : rows;
    const bool all = (a.mode == 0 && a.nstar >= (float)a.NK) || a.mode == 2 || (a.mode == 1 && a.kstar >= a.NK);
    if (all || (a.mode == 1 && a.kstar <= 0)) {
      sel_all_kernel<<<nlists, 256, 0, st>>>(a, all ? 1 : 0);
    } else {
      // waves per list: one up to 20 blocks per layout thread (80 score registers
      // per lane), else two or four with at most 16 (the multi-wave kernel keeps
      // a few more registers live); P is then exactly an instantiated chunk size
      const int wpl = a.NK <= 5120 ? 1 : (a.NK <= 8192 ? 2 : 4);
      const int P = 4 * ((a.NK + 1024 * wpl - 1) / (1024 * wpl));
      const bool sip = a.mode == 0;
#define ABSA_SR(PP, WW)                                                                                   \
  do {                                                                                                    \
    const dim3 grid(WW == 1 ? (nlists + SR_WAVES - 1) / SR_WAVES : nlists);                               \
    const int nt = 64 * (WW == 1 ? SR_WAVES : WW);                                                        \
    if (sip) sip_rows_kernel<PP, SR_SIP, WW><<<grid, nt, 0, st>>>(a, nlists, NKs);                        \
    else sip_rows_kernel<PP, SR_TOPK, WW><<<grid, nt, 0, st>>>(a, nlists, NKs);                           \
  } while (0)
      if (wpl == 1) {
        switch (P) {
          case 4: ABSA_SR(4, 1); break;
          case 8: ABSA_SR(8, 1); break;
          case 12: ABSA_SR(12, 1); break;
          case 16: ABSA_SR(16, 1); break;
          case 20: ABSA_SR(20, 1); break;
          default: return hipErrorInvalidValue;
        }
      } else if (wpl == 2) {  // 5120 < NK <= 8192
        switch (P) {
          case 12: ABSA_SR(12, 2); break;
          case 16: ABSA_SR(16, 2); break;
          default: return hipErrorInvalidValue;
        }
      } else {  // 8192 < NK <= 12288
        if (P != 12) return hipErrorInvalidValue;
        ABSA_SR(12, 4);
      }
#undef ABSA_SR
    }
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && !a.per_cluster) e = mark();
    if (e != hipSuccess) return e;
  }
  // union of the per-cluster lists
  if (a.per_cluster) {
    cluster_union_kernel<<<rows, SIP_NT, (size_t)a.NK * sizeof(uint32_t), st>>>(
        a.count, a.kv_idx, a.inv_pi, a.cap, a.C, a.NK, a.ucount, a.uidx, a.uw, a.ucap, 0, 0);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = mark();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t configure_select_kernels() {
  // (nothing to configure: the selection kernels use static LDS only)
  return hipSuccess;
}

}  // namespace absa
