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
// kbar^T[bh][c][b] = (1/n_b) sum_{valid keys of block b} K[bh][key][c], and the
// same means block-major as bf16 head and tail, hi = bf16(kbar), lo =
// bf16(kbar - hi) (kbh[bh][b][c], then kbl at kbh + BH NKp D), the operands of
// the logit product.  Padding blocks (b >= NK) are 0.
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
  float* dst = kbarT + (size_t)bh * D * NKp + b0;
  for (int idx = t; idx < D * 64; idx += 256) {
    const int cc = idx >> 6, bl = idx & 63;
    dst[(size_t)cc * NKp + bl] = tile[cc][bl];
  }
  const size_t tail = (size_t)gridDim.y * NKp * D;
  for (int idx = t; idx < 64 * D / 8; idx += 256) {
    const int bl = idx / (D / 8), c8 = idx % (D / 8);
    bf16x8 hv, lv;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = tile[c8 * 8 + e][bl];
      const __bf16 hi = (__bf16)x;
      hv[e] = hi;
      lv[e] = (__bf16)(x - (float)hi);
    }
    const size_t o = ((size_t)bh * NKp + b0 + bl) * D + c8 * 8;
    *reinterpret_cast<bf16x8*>(kbh + o) = hv;
    *reinterpret_cast<bf16x8*>(kbh + tail + o) = lv;
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
// and mu . kbar is formed as hi.hi' + hi.lo' + lo.hi' in one fp32 accumulator:
// the dropped lo.lo' and remainder terms are below 2^-15 of each product, and
// operands that bf16 holds exactly (lo = 0) give the exact fp32 dot product.
// Workgroup = 4 waves x 32 centroids; a wave keeps its centroids' heads and
// tails as A operands in registers and streams 32-block tiles of the means'
// heads and tails (split once, by K1) through LDS.  Logit rows have NKp
// entries (the padding holds -inf and is never read); a wave turns its 32 x 32
// logits around in LDS so that each lane stores 16 contiguous bytes.
// Grid (ceil(M/128), BH, nsplit): split z covers a contiguous range of 32-block
// tiles.
template <int D>
__global__ __launch_bounds__(256) void ibcs_logit_kernel(const uint16_t* __restrict__ kbh,
                                                         const float* __restrict__ mu,
                                                         float* __restrict__ logit,
                                                         float2* __restrict__ mz, int M, int NK,
                                                         int NKp, int L, int Bk, int tiles_per_split,
                                                         float alpha) {
  constexpr int KS = D / 16;  // k-steps of 16 dims
  // [buffer][block row][D] bf16, 16-byte chunks swizzled by row as in the
  // attention kernels' K tiles, so the 32 rows a k-step reads are conflict-free
  __shared__ __attribute__((aligned(16))) unsigned char khi[2][32 * D * 2], klo[2][32 * D * 2];
  constexpr int LPS = 40;  // row stride of a wave's logit patch (the two half-waves' writes hit disjoint banks)
  __shared__ __attribute__((aligned(16))) float lpatch[4][32 * LPS];
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform (scalar) index
  const int h = lane >> 5, n = lane & 31;
  const int bh = blockIdx.y;
  const int m0 = blockIdx.x * 128 + w * 32;
  const int tile0 = blockIdx.z * tiles_per_split;
  const int ntile_all = NKp / 32;
  const int tile1 = min(ntile_all, tile0 + tiles_per_split);
  if (tile0 >= tile1) return;

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
  // 16-byte chunks of a tile: NCK per operand (head, tail), NST per thread
  constexpr int NCK = 32 * D / 8, NST = 2 * NCK / 256;
  const uint16_t* kb = kbh + (size_t)bh * NKp * D;
  const size_t tail = (size_t)gridDim.y * NKp * D;
  // two register stages: the global loads of a tile are issued two tiles
  // ahead of its store into LDS, so their latency spans two tile periods
  u32x4 stA[NST], stB[NST];
  auto fetch = [&](u32x4 (&stage)[NST], int tile) {
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      const int idx = t + 256 * i, rem = idx % NCK;
      stage[i] = *reinterpret_cast<const u32x4*>(kb + (idx >= NCK ? tail : 0) + (size_t)(tile * 32) * D + rem * 8);
    }
  };
  auto put = [&](const u32x4 (&stage)[NST], int buf) {
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      const int idx = t + 256 * i, rem = idx % NCK;
      const int off = k_off<D>(rem / (D / 8), rem % (D / 8));
      *reinterpret_cast<u32x4*>(idx >= NCK ? &klo[buf][off] : &khi[buf][off]) = stage[i];
    }
  };
  fetch(stA, tile0);
  put(stA, 0);
  if (tile0 + 1 < tile1) fetch(stA, tile0 + 1);
  // this wave's output window: logit rows m0 .. m0+31 (those below M) of the head
  const int rows_here = max(0, min(32, M - m0));
  const uint64_t obase = (uint64_t)(logit + ((size_t)bh * M + (rows_here > 0 ? m0 : 0)) * NKp);
  const uint32_t obase_lo = __builtin_amdgcn_readfirstlane((uint32_t)obase);
  const uint32_t obase_hi = __builtin_amdgcn_readfirstlane((uint32_t)(obase >> 32));
  const int obytes = __builtin_amdgcn_readfirstlane(rows_here * NKp * 4);
  float* const lp = lpatch[w];
  const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(((uint64_t)obase_hi << 32) | obase_lo), 0, obytes, 0x00020000);
  // running max m and normaliser Z = sum nk 2^(l - m) of the 16 centroids this
  // lane sees (terms more than 64 octaves below the max dropped)
  float rm[16], rz[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) { rm[r] = -INFINITY; rz[r] = 0.f; }
  // one tile: sput holds tile + 1 (stored into the other LDS buffer at the
  // end), sfetch receives tile + 2; the loop alternates the two stages
  auto body = [&](int tile, const u32x4 (&sput)[NST], u32x4 (&sfetch)[NST]) {
    const int buf = (tile - tile0) & 1;
    __syncthreads();
    if (tile + 2 < tile1) fetch(sfetch, tile + 2);
    // B operands: lane (h, n) reads block n, channels 16 s + 8 h .. +7
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    // operand reads two k-steps ahead of their products (fewer live registers)
    bf16x8 bhi[KS], blo[KS];
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      const int off = k_off<D>(n, 2 * s2 + h);
      bhi[s2] = *reinterpret_cast<const bf16x8*>(&khi[buf][off]);
      blo[s2] = *reinterpret_cast<const bf16x8*>(&klo[buf][off]);
    }
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[s2], bhi[s2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[s2], blo[s2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo[s2], bhi[s2], acc, 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
      if (s2 + 2 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    // Online (m, Z): with d = |m - l| only one of the two factors 2^(m - max)
    // and 2^(l - max) differs from 1, so one exp2 per logit suffices.  Padding
    // blocks (b >= NK) enter as l = -inf, which changes neither m nor Z; stores
    // of rows >= M fall outside the window and are dropped.
    const int b = tile * 32 + n;
    const bool bv = b < NK;
    const float nk = (float)min(Bk, L - b * Bk);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float l = bv ? alpha * acc[r] : -INFINITY;
      lp[(8 * (r >> 2) + 4 * h + (r & 3)) * LPS + n] = l;
      const float dd = fabsf(rm[r] - l);
      const float e = dd <= 64.f ? exp2_split(-dd) : 0.f;
      const bool up = l > rm[r];
      rz[r] = fmaf(rz[r], up ? e : 1.f, up ? nk : nk * e);
      rm[r] = up ? l : rm[r];
    }
    // lane i stores blocks 4 (i % 8) .. +3 of patch rows 8 q + i / 8
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int pr = 8 * q + (lane >> 3), c4 = 4 * (lane & 7);
      const u32x4 v = *reinterpret_cast<const u32x4*>(&lp[pr * LPS + c4]);
      __builtin_amdgcn_raw_buffer_store_b128(v, ors, (pr * NKp + tile * 32 + c4) * 4, 0, 0);
    }
    if (tile + 1 < tile1) put(sput, buf ^ 1);
  };
#pragma unroll 1
  for (int tile = tile0; tile < tile1; tile += 2) {
    body(tile, stA, stB);
    if (tile + 1 < tile1) body(tile + 1, stB, stA);
  }
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
    if (n == 0 && m < M) mz[((size_t)bh * M + m) * gridDim.z + blockIdx.z] = make_float2(rm[r], rz[r]);
  }
}

// ============================================================================= K3
// One workgroup per row: inclusion probabilities by iterative capping, Philox
// Bernoulli draws (or top-k / all), and compaction into the row's list.
constexpr int SIP_NT = 256;

// Capping rounds of the SIP inclusion probabilities over one thread's chunk of
// n <= PM block scores s[b0 .. b0+n).  The chunk stays in registers; each round
// caps the free blocks with s R >= S_U and, in the same block reduction, forms
// the sum over the blocks still free, which is the next round's S_U (the same
// set, summed in the same order, as a fresh sum over the free blocks).  On
// return flag[] holds 1 for capped, 0 for free (s > 0), 2 for zero blocks, and
// R, S_U the remaining budget and free-score sum of the last round.
template <int PM>
__device__ __forceinline__ void sip_capping(const float* s, int b0, int n, float& R, float& S_U, unsigned char* flag,
                                            float* redf, int* redi) {
  float sv[PM];
  uint64_t freem = 0ull, capm = 0ull;
  float part = 0.f;
  int nfree = 0;
#pragma unroll
  for (int e = 0; e < PM; ++e) {
    sv[e] = (e < n) ? s[b0 + e] : 0.f;
    if (sv[e] > 0.f) {
      freem |= 1ull << e;
      part += sv[e];
      ++nfree;
    }
  }
  int parity = 0;
  block_total2<SIP_NT>(part, nfree, redf, redi, parity);
  S_U = part;
#pragma unroll 1
  while (nfree > 0) {
    int ncap = 0;
    part = 0.f;
#pragma unroll
    for (int e = 0; e < PM; ++e) {
      if ((freem >> e) & 1ull) {
        if (__fmul_rn(sv[e], R) >= S_U) {
          freem &= ~(1ull << e);
          capm |= 1ull << e;
          ++ncap;
        } else {
          part += sv[e];
        }
      }
    }
    parity ^= 1;
    block_total2<SIP_NT>(part, ncap, redf, redi, parity);
    if (ncap == 0) break;
    S_U = part;
    R -= (float)ncap;
    nfree -= ncap;
  }
#pragma unroll
  for (int e = 0; e < PM; ++e)
    if (e < n) flag[b0 + e] = ((capm >> e) & 1ull) ? 1 : (sv[e] > 0.f ? 0 : 2);
}

template <int C>
__global__ __launch_bounds__(SIP_NT) void sip_kernel(const float* __restrict__ logit,
                                                     const float2* __restrict__ mz, int nsplit,
                                                     const int* __restrict__ nj,
                                                     float* __restrict__ s_out, int L, int Bq, int Bk,
                                                     int NK, int NKp, int NQ,
                                                     float nstar, int kstar, int mode, uint32_t key0,
                                                     uint32_t key1, uint32_t ctr3,
                                                     int32_t* __restrict__ count_out,
                                                     int32_t* __restrict__ kv_idx,
                                                     float* __restrict__ inv_pi, int cap,
                                                     float* __restrict__ pi_out, int per_cluster) {
  extern __shared__ float s[];                      // [NK]
  unsigned char* flag = reinterpret_cast<unsigned char*>(s + NK);  // [NK]
  __shared__ float redf[2 * (SIP_NT / 64)];
  __shared__ int redi[2 * (SIP_NT / 64)];
  const int t = threadIdx.x;
  const int row = blockIdx.x;
  const int bh = row / NQ, i = row % NQ;
  // Per-cluster lists: workgroup (row, j) samples cluster j alone (its own block
  // distribution, the full budget, Philox counter word i C + j) into list row C + j;
  // a cluster without members gets an empty list.
  const int jsel = per_cluster ? (int)blockIdx.y : -1;
  const int orow = per_cluster ? row * C + jsel : row;
  if (per_cluster && nj[(size_t)row * C + jsel] == 0) {
    if (t == 0) count_out[orow] = 0;
    return;
  }

  // ---- IBCS scores of this row from its logits: per centroid the max m_j and
  // the normaliser Z_j = sum_b nk_b 2^(l_jb - m_j) (terms below 2^-64 of the
  // max dropped; combined from the logit kernel's per-split partials), then
  // s_b = sum_j (n_j/n) nk_b 2^(l_jb - m_j) / Z_j.
  {
    const float* lrow = logit + (size_t)row * C * NKp;
    __shared__ float coef_s[C], mj_s[C];
    if (t < C) {
      const float2* pz = mz + ((size_t)row * C + t) * nsplit;
      float m = -INFINITY;
      for (int z = 0; z < nsplit; ++z) m = fmaxf(m, pz[z].x);
      float zs = 0.f;
      for (int z = 0; z < nsplit; ++z) {
        const float d = pz[z].x - m;
        if (d >= -64.f) zs = fmaf(pz[z].y, exp2_split(d), zs);
      }
      const int n = min(Bq, L - i * Bq);
      const int cnt = nj[(size_t)row * C + t];
      mj_s[t] = m;
      if (per_cluster)
        coef_s[t] = (t == jsel) ? __fdiv_rn(1.f, zs) : 0.f;
      else
        coef_s[t] = (cnt > 0) ? __fdiv_rn(__fdiv_rn((float)cnt, (float)n), zs) : 0.f;
    }
    __syncthreads();
    float mj[C], coef[C];
#pragma unroll
    for (int j = 0; j < C; ++j) { mj[j] = mj_s[j]; coef[j] = coef_s[j]; }
    constexpr int U = 8;  // blocks per batch: U*C loads in flight
    float* srow_out = s_out + (size_t)orow * NK;
#pragma unroll 1
    for (int b0 = t; b0 < NK; b0 += U * SIP_NT) {
      float lv[U][C];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < C; ++j) {
          const int b = b0 + u * SIP_NT;
          // (a centroid with coefficient 0 -- an empty cluster, or another
          // cluster's in a per-cluster sample -- is not read at all)
          lv[u][j] = (b < NK && coef[j] != 0.f) ? lrow[(size_t)j * NKp + b] : -INFINITY;
        }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int b = b0 + u * SIP_NT;
        if (b >= NK) break;
        const float nk = (float)min(Bk, L - b * Bk);
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < C; ++j) {
          const float dl = lv[u][j] - mj[j];
          if (dl >= -64.f && coef[j] != 0.f) acc = fmaf(coef[j], nk * exp2_split(dl), acc);
        }
        s[b] = acc;
        srow_out[b] = acc;
      }
    }
  }
  // contiguous chunk of P blocks per thread, P a multiple of 4
  const int P = ((NK + SIP_NT * 4 - 1) / (SIP_NT * 4)) * 4;
  const int b0 = min(NK, t * P), b1 = min(NK, b0 + P);
  __syncthreads();

  // flag: 0 free (pi = s R / S_U), 1 capped (pi = 1), 2 zero (pi = 0), 3 kept, 4 dropped
  float R = nstar, S_U = 1.f;
  if (mode == 0) {
    if (nstar >= (float)NK) {
      for (int b = b0; b < b1; ++b) flag[b] = 1;
    } else {
      const int n = b1 - b0;
      if (P <= 16) sip_capping<16>(s, b0, n, R, S_U, flag, redf, redi);
      else if (P <= 24) sip_capping<24>(s, b0, n, R, S_U, flag, redf, redi);
      else if (P <= 32) sip_capping<32>(s, b0, n, R, S_U, flag, redf, redi);
      else sip_capping<48>(s, b0, n, R, S_U, flag, redf, redi);
    }
  } else if (mode == 1) {
    // top-k*: largest bit pattern T with #{s >= T} >= k*, then the lowest-index ties
    for (int b = b0; b < b1; ++b) flag[b] = 4;
    if (kstar >= NK) {
      for (int b = b0; b < b1; ++b) flag[b] = 3;
    } else if (kstar > 0) {
      uint32_t lo = 0u, hi = 0x7F800001u;
#pragma unroll 1
      while (hi - lo > 1u) {
        const uint32_t mid = lo + ((hi - lo) >> 1);
        int c = 0;
        for (int b = b0; b < b1; ++b) c += (__float_as_uint(s[b]) >= mid);
        c = block_sum_i<SIP_NT>(c, redi);
        if (c >= kstar) lo = mid; else hi = mid;
      }
      int gt = 0, eq = 0;
      for (int b = b0; b < b1; ++b) {
        const uint32_t u = __float_as_uint(s[b]);
        gt += (u > lo);
        eq += (u == lo);
      }
      const int ngt = block_sum_i<SIP_NT>(gt, redi);
      int tot;
      int rank = block_exclusive_scan<SIP_NT>(eq, redi, tot);
      const int need = kstar - ngt;
      for (int b = b0; b < b1; ++b) {
        const uint32_t u = __float_as_uint(s[b]);
        if (u > lo) flag[b] = 3;
        else if (u == lo) { if (rank < need) flag[b] = 3; ++rank; }
      }
    }
  } else {
    for (int b = b0; b < b1; ++b) flag[b] = 3;
  }

  // probabilities, draws, weights
  int nkept = 0;
  for (int g = b0; g < b1; g += 4) {
    philox_u4 x = {0u, 0u, 0u, 0u};
    const uint32_t ctr1 = per_cluster ? (uint32_t)(i * C + jsel) : (uint32_t)i;
    if (mode == 0) x = philox4x32_10({(uint32_t)(g >> 2), ctr1, (uint32_t)bh, ctr3}, key0, key1);
    const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int b = g + e;
      if (b < b1) {
        float p;
        if (mode == 0) {
          const int f = flag[b];
          p = (f == 1) ? 1.f : (f == 2) ? 0.f : __fdiv_rn(__fmul_rn(s[b], R), S_U);
          const float u = (float)(xw[e] >> 8) * 0x1p-24f;
          const bool keep = u < p;
          flag[b] = keep ? 3 : 4;
          s[b] = p;  // s is no longer needed: keep pi for the weight
        } else {
          p = (flag[b] == 3) ? 1.f : 0.f;
          s[b] = p;
        }
        if (pi_out) pi_out[(size_t)row * NK + b] = p;
        nkept += (flag[b] == 3);
      }
    }
  }
  int total;
  int off = block_exclusive_scan<SIP_NT>(nkept, redi, total);
  int32_t* idx_row = kv_idx + (size_t)orow * cap;
  float* w_row = inv_pi + (size_t)orow * cap;
  for (int b = b0; b < b1; ++b) {
    if (flag[b] == 3) {
      idx_row[off] = b;
      w_row[off] = (mode == 0) ? __frcp_rn(s[b]) : 1.f;
      ++off;
    }
  }
  if (t == 0) count_out[orow] = total;
}

// ============================================================================= per-cluster union
// One workgroup per row: the ascending union of the row's C cluster lists and
// the weight of every (entry, cluster) pair, 0 where the cluster did not draw
// the block.  LDS holds one word per KV block: the cluster mask in the low 8
// bits, the union position above it.  The weight rows are zeroed with
// contiguous stores, then each cluster's drawn weights are scattered in.
__global__ __launch_bounds__(SIP_NT) void cluster_union_kernel(const int32_t* __restrict__ ccount,
                                                               const int32_t* __restrict__ cidx,
                                                               const float* __restrict__ cw, int ccap, int C,
                                                               int NK, int32_t* __restrict__ ucount,
                                                               int32_t* __restrict__ uidx, float* __restrict__ uw,
                                                               int ucap) {
  extern __shared__ uint32_t slot[];  // [NK]
  __shared__ int redi[2 * (SIP_NT / 64)];
  const int t = threadIdx.x;
  const size_t row = blockIdx.x;
  for (int b = t; b < NK; b += SIP_NT) slot[b] = 0u;
  __syncthreads();
  for (int j = 0; j < C; ++j) {
    const int n = min(ccount[row * C + j], ccap);
    const int32_t* li = cidx + (row * C + j) * ccap;
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
    const int n = min(ccount[row * C + j], ccap);
    const int32_t* li = cidx + (row * C + j) * ccap;
    const float* lw = cw + (row * C + j) * ccap;
    for (int e = t; e < n; e += SIP_NT) {
      const int b = li[e];
      if ((unsigned)b < (unsigned)NK) wrow[(size_t)(slot[b] >> 8) * C + j] = lw[e];
    }
  }
  if (t == 0) ucount[row] = total;
}

// ============================================================================= launchers
hipError_t launch_select(const SelectLaunch& a, hipStream_t st) {
  const int BH = a.B * a.H;
  const int rows = BH * a.NQ;
  // K1
  {
    dim3 grid(a.NKp / 64, BH);
    if (a.d == 128)
      kv_block_mean_kernel<128><<<grid, 256, 0, st>>>(a.k, a.kbarT, a.kbh, a.L, a.Bk, a.NK, a.NKp);
    else
      kv_block_mean_kernel<64><<<grid, 256, 0, st>>>(a.k, a.kbarT, a.kbh, a.L, a.Bk, a.NK, a.NKp);
    hipError_t e = hipGetLastError();
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
    if (e != hipSuccess) return e;
  }
  // K2b
  {
    const int M = a.NQ * a.C;
    const int mtiles = (M + 127) / 128;
    int per;
    const int nsplit = logit_splits(a.NQ, a.C, BH, a.NKp, &per);
    dim3 grid(mtiles, BH, nsplit);
    if (a.d == 128)
      ibcs_logit_kernel<128><<<grid, 256, 0, st>>>(a.kbh, a.mu, a.logit, a.mz, M, a.NK, a.NKp, a.L,
                                                   a.Bk, per, a.alpha);
    else
      ibcs_logit_kernel<64><<<grid, 256, 0, st>>>(a.kbh, a.mu, a.logit, a.mz, M, a.NK, a.NKp, a.L,
                                                  a.Bk, per, a.alpha);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // K3
  {
    int per;
    const int nsplit = logit_splits(a.NQ, a.C, BH, a.NKp, &per);
    const size_t lds = (size_t)a.NK * (sizeof(float) + 1);
    const dim3 sgrid(rows, a.per_cluster ? a.C : 1);
#define ABSA_SIP(CC)                                                                                   \
  sip_kernel<CC><<<sgrid, SIP_NT, lds, st>>>(a.logit, a.mz, nsplit, a.nj, a.s, a.L, a.Bq, a.Bk, a.NK,  \
                                             a.NKp, a.NQ, a.nstar,                                              \
                                             a.kstar, a.mode, a.key0, a.key1, a.ctr3, a.count, a.kv_idx, \
                                             a.inv_pi, a.cap, a.pi_out, a.per_cluster)
    switch (a.C) {
      case 1: ABSA_SIP(1); break;
      case 2: ABSA_SIP(2); break;
      case 4: ABSA_SIP(4); break;
      default: ABSA_SIP(8); break;
    }
#undef ABSA_SIP
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // union of the per-cluster lists
  if (a.per_cluster) {
    cluster_union_kernel<<<rows, SIP_NT, (size_t)a.NK * sizeof(uint32_t), st>>>(
        a.count, a.kv_idx, a.inv_pi, a.cap, a.C, a.NK, a.ucount, a.uidx, a.uw, a.ucap);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t configure_select_kernels() {
  // The SIP kernel keeps one row of scores and flags in LDS: up to 60 KB.
  hipError_t e;
#define ABSA_ATTR(CC)                                                                   \
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&sip_kernel<CC>),              \
                          hipFuncAttributeMaxDynamicSharedMemorySize, 12288 * 5);      \
  if (e != hipSuccess) return e;
  ABSA_ATTR(1) ABSA_ATTR(2) ABSA_ATTR(4) ABSA_ATTR(8)
#undef ABSA_ATTR
  return hipSuccess;
}

}  // namespace absa
