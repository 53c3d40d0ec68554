// Block selection kernels for gfx950: KV block means, IBCS in-block k-means,
// IBCS block scoring and SIP sampling (AB-Attention page, section "AB-Attention
// ve Üç Temel Yeniliği", IBCS and SIP items).  The rules each kernel follows are
// listed in absa.h.  Everything is fp32 with correctly rounded divisions, so on
// inputs whose intermediates are exactly representable the lists and
// probabilities equal those of an exact computation.
#include "absa_device.h"
#include "absa_launch.h"

// No implicit multiply-add fusion: every product below is rounded on its own,
// as the selection arithmetic contract requires; fused steps are explicit fmaf.
#pragma clang fp contract(off)

namespace absa {

// 2^x, exact whenever the result is representable and x is an integer: the
// integer part goes through ldexp, only the fractional part through v_exp_f32.
__device__ __forceinline__ float exp2_split(float x) {
  const float fl = floorf(x);
  return ldexpf(__builtin_amdgcn_exp2f(x - fl), (int)fl);
}

// ============================================================================= K1
// kbar^T[bh][c][b] = (1/n_b) sum_{valid keys of block b} K[bh][key][c].
// Grid (NKp/64, BH), 256 threads; a workgroup produces 64 blocks x D dims.
template <int D>
__global__ __launch_bounds__(256) void kv_block_mean_kernel(const uint16_t* __restrict__ k,
                                                            float* __restrict__ kbarT, int L, int Bk,
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
      for (int r = 0; r < n; ++r) {
        const uint4 w = src[(size_t)r * (D / 8)];
        float lo, hi;
        unpack_bf16x2(w.x, lo, hi); acc[0] += lo; acc[1] += hi;
        unpack_bf16x2(w.y, lo, hi); acc[2] += lo; acc[3] += hi;
        unpack_bf16x2(w.z, lo, hi); acc[4] += lo; acc[5] += hi;
        unpack_bf16x2(w.w, lo, hi); acc[6] += lo; acc[7] += hi;
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
}

// ============================================================================= K2a
// Lloyd k-means of one query block (one workgroup per row).  Queries stay in
// token order; centroids start at members floor(j n / C); each step assigns
// every query to its nearest centroid (squared Euclidean, ties to the lowest
// j) and moves each non-empty centroid to the mean of its members.
template <int D>
__global__ __launch_bounds__(256) void ibcs_kmeans_kernel(const uint16_t* __restrict__ q,
                                                          float* __restrict__ mu_out,
                                                          int* __restrict__ nj_out, int L, int Bq,
                                                          int NQ, int C, int Tk) {
  constexpr int XS = D / 2 + 1;  // row stride in dwords (bf16 pairs), odd -> conflict-free
  constexpr int G = 256 / D;     // query groups in the update step
  __shared__ uint32_t X[128 * XS];
  __shared__ float mu[8][D];
  __shared__ float dpart[2][128][8];
  __shared__ float upd[G][8][D];
  __shared__ int label[128];
  __shared__ int cnt[8];

  const int t = threadIdx.x;
  const int row = blockIdx.x;
  const int bh = row / NQ, i = row % NQ;
  const int q0 = i * Bq;
  const int n = min(Bq, L - q0);
  const uint32_t* src = reinterpret_cast<const uint32_t*>(q + ((size_t)bh * L + q0) * D);
  for (int idx = t; idx < n * (D / 2); idx += 256) {
    const int qq = idx / (D / 2), cp = idx % (D / 2);
    X[qq * XS + cp] = src[idx];
  }
  __syncthreads();
  for (int idx = t; idx < C * D; idx += 256) {
    const int j = idx / D, c = idx % D;
    const int m = (j * n) / C;
    const uint32_t w = X[m * XS + (c >> 1)];
    mu[j][c] = (c & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
  }
  __syncthreads();

#pragma unroll 1
  for (int step = 0; step < Tk; ++step) {
    // assign: thread -> (query qq, half hf of the dims)
    {
      const int qq = t & 127, hf = t >> 7;
      if (qq < n) {
        float dist[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) dist[j] = 0.f;
        const uint32_t* xr = X + qq * XS + hf * (D / 4);
#pragma unroll 4
        for (int cp = 0; cp < D / 4; ++cp) {
          float x0, x1;
          unpack_bf16x2(xr[cp], x0, x1);
          const int c = hf * (D / 2) + 2 * cp;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if (j < C) {
              const float d0 = x0 - mu[j][c], d1 = x1 - mu[j][c + 1];
              dist[j] = fmaf(d0, d0, dist[j]);
              dist[j] = fmaf(d1, d1, dist[j]);
            }
          }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j < C) dpart[hf][qq][j] = dist[j];
      }
    }
    if (t < 8) cnt[t] = 0;
    __syncthreads();
    if (t < n) {
      int best = 0;
      float bd = dpart[0][t][0] + dpart[1][t][0];
      for (int j = 1; j < C; ++j) {
        const float dj = dpart[0][t][j] + dpart[1][t][j];
        if (dj < bd) { bd = dj; best = j; }
      }
      label[t] = best;
      atomicAdd(&cnt[best], 1);
    }
    __syncthreads();
    // update: thread -> (group g of queries, dim c)
    {
      const int c = t % D, g = t / D;
      const int per = (n + G - 1) / G;
      const int qa = g * per, qb = min(n, qa + per);
      float sum[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) sum[j] = 0.f;
      for (int qq = qa; qq < qb; ++qq) {
        const uint32_t w = X[qq * XS + (c >> 1)];
        const float x = (c & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
        const int lb = label[qq];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j == lb) sum[j] += x;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) upd[g][j][c] = sum[j];
    }
    __syncthreads();
    for (int idx = t; idx < C * D; idx += 256) {
      const int j = idx / D, c = idx % D;
      if (cnt[j] > 0) {
        float s = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) s += upd[g][j][c];
        mu[j][c] = __fdiv_rn(s, (float)cnt[j]);
      }
    }
    __syncthreads();
  }
  float* mo = mu_out + (size_t)row * C * D;
  for (int idx = t; idx < C * D; idx += 256) mo[idx] = mu[idx / D][idx % D];
  if (t < C) nj_out[(size_t)row * C + t] = (Tk > 0) ? cnt[t] : 0;
}

// ============================================================================= K2b
// Scores of every KV block for RPW = 128/C rows of one head (a 128-centroid x
// 64-block tile per step).  Pass 1 finds each centroid's max logit and its
// normaliser Z_j online; pass 2 recomputes the logits and writes
// s_b = sum_j (n_j/n) nk_b 2^(l_jb - m_j) / Z_j (0 below the -64 floor).
// Thread micro-tile: 8 centroids (8/C rows) x 4 blocks.
template <int D, int C>
__global__ __launch_bounds__(256) void ibcs_score_kernel(const float* __restrict__ kbarT,
                                                         const float* __restrict__ mu,
                                                         const int* __restrict__ nj,
                                                         float* __restrict__ s_out, int L, int Bk,
                                                         int Bq, int NQ, int NK, int NKp,
                                                         float alpha) {
  constexpr int RPW = 128 / C;
  constexpr int RPT = 8 / C;  // rows per thread
  extern __shared__ float smem[];
  float* muT = smem;               // [D][128]
  float* kT = smem + D * 128;      // [D][64]
  const int t = threadIdx.x;
  const int tb = t & 15, tc = t >> 4;
  const int bh = blockIdx.y;
  const int r0 = blockIdx.x * RPW;

  for (int idx = t; idx < D * 128; idx += 256) {
    const int cv = idx & 127, c = idx >> 7;
    const int r = r0 + cv / C;
    muT[c * 128 + cv] = (r < NQ) ? mu[((size_t)(bh * NQ + r) * C + (cv % C)) * D + c] : 0.f;
  }
  const float* kb = kbarT + (size_t)bh * D * NKp;
  const int ntiles = NKp / 64;

  float m_run[8], z_run[8];
#pragma unroll
  for (int a = 0; a < 8; ++a) { m_run[a] = -INFINITY; z_run[a] = 0.f; }

  auto load_tile = [&](int tile) {
    __syncthreads();
    for (int idx = t; idx < D * 16; idx += 256) {
      const int c = idx >> 4, b4 = idx & 15;
      *reinterpret_cast<float4*>(kT + c * 64 + b4 * 4) =
          *reinterpret_cast<const float4*>(kb + (size_t)c * NKp + tile * 64 + b4 * 4);
    }
    __syncthreads();
  };
  auto compute = [&](float (&acc)[8][4]) {
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;
#pragma unroll 4
    for (int c = 0; c < D; ++c) {
      const float4 m0 = *reinterpret_cast<const float4*>(muT + c * 128 + tc * 8);
      const float4 m1 = *reinterpret_cast<const float4*>(muT + c * 128 + tc * 8 + 4);
      const float4 kv = *reinterpret_cast<const float4*>(kT + c * 64 + tb * 4);
      const float mv[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
      const float kk[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fmaf(mv[a], kk[b], acc[a][b]);
    }
  };

  // ---- pass 1: per-centroid max and normaliser
#pragma unroll 1
  for (int tile = 0; tile < ntiles; ++tile) {
    load_tile(tile);
    float acc[8][4];
    compute(acc);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int blk = tile * 64 + tb * 4 + b;
      if (blk < NK) {
        const float nk = (float)min(Bk, L - blk * Bk);
#pragma unroll
        for (int a = 0; a < 8; ++a) {
          const float l = alpha * acc[a][b];
          if (l > m_run[a]) {
            z_run[a] = (m_run[a] - l >= -64.f) ? fmaf(z_run[a], exp2_split(m_run[a] - l), nk) : nk;
            m_run[a] = l;
          } else if (l - m_run[a] >= -64.f) {
            z_run[a] = fmaf(nk, exp2_split(l - m_run[a]), z_run[a]);
          }
        }
      }
    }
  }
  // combine the 16 block-groups that share these centroids (lanes 16k..16k+15)
#pragma unroll
  for (int a = 0; a < 8; ++a) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const float m2 = __shfl_xor(m_run[a], o, 64);
      const float z2 = __shfl_xor(z_run[a], o, 64);
      const float m = fmaxf(m_run[a], m2);
      float z = 0.f;
      if (m_run[a] - m >= -64.f) z += z_run[a] * exp2_split(m_run[a] - m);
      if (m2 - m >= -64.f) z += z2 * exp2_split(m2 - m);
      m_run[a] = m;
      z_run[a] = z;
    }
  }
  // coefficient (n_j / n) / Z_j of each of this thread's centroids
  float coef[8];
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const int cv = tc * 8 + a;
    const int r = r0 + cv / C;
    coef[a] = 0.f;
    if (r < NQ) {
      const int n = min(Bq, L - r * Bq);
      const int cnt = nj[(size_t)(bh * NQ + r) * C + (cv % C)];
      if (cnt > 0) coef[a] = __fdiv_rn(__fdiv_rn((float)cnt, (float)n), z_run[a]);
    }
  }
  // ---- pass 2: scores
#pragma unroll 1
  for (int tile = 0; tile < ntiles; ++tile) {
    load_tile(tile);
    float acc[8][4];
    compute(acc);
#pragma unroll
    for (int rr = 0; rr < RPT; ++rr) {
      const int r = r0 + (tc * 8) / C + rr;
      float sv[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int blk = tile * 64 + tb * 4 + b;
        const float nk = (blk < NK) ? (float)min(Bk, L - blk * Bk) : 0.f;
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < C; ++j) {
          const int a = rr * C + j;
          const float dl = alpha * acc[a][b] - m_run[a];
          if (dl >= -64.f && coef[a] != 0.f) s = fmaf(coef[a], nk * exp2_split(dl), s);
        }
        sv[b] = s;
      }
      if (r < NQ) {
        float* dst = s_out + (size_t)(bh * NQ + r) * NK + tile * 64 + tb * 4;
        const int blk0 = tile * 64 + tb * 4;
#pragma unroll
        for (int b = 0; b < 4; ++b)
          if (blk0 + b < NK) dst[b] = sv[b];
      }
    }
  }
}

// ============================================================================= K3
// One workgroup per row: inclusion probabilities by iterative capping, Philox
// Bernoulli draws (or top-k / all), and compaction into the row's list.
constexpr int SIP_NT = 256;

__global__ __launch_bounds__(SIP_NT) void sip_kernel(const float* __restrict__ s_all, int NK, int NQ,
                                                     float nstar, int kstar, int mode, uint32_t key0,
                                                     uint32_t key1, uint32_t ctr3,
                                                     int32_t* __restrict__ count_out,
                                                     int32_t* __restrict__ kv_idx,
                                                     float* __restrict__ inv_pi, int cap,
                                                     float* __restrict__ pi_out) {
  extern __shared__ float s[];                      // [NK]
  unsigned char* flag = reinterpret_cast<unsigned char*>(s + NK);  // [NK]
  __shared__ float redf[SIP_NT / 64];
  __shared__ int redi[SIP_NT / 64];
  const int t = threadIdx.x;
  const int row = blockIdx.x;
  const int bh = row / NQ, i = row % NQ;
  const float* srow = s_all + (size_t)row * NK;
  for (int b = t; b < NK; b += SIP_NT) s[b] = srow[b];
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
      for (int b = b0; b < b1; ++b) flag[b] = (s[b] > 0.f) ? 0 : 2;
      int nfree = 0;
      for (int b = b0; b < b1; ++b) nfree += (flag[b] == 0);
      nfree = block_sum_i<SIP_NT>(nfree, redi);
#pragma unroll 1
      while (nfree > 0) {
        float part = 0.f;
        for (int b = b0; b < b1; ++b)
          if (flag[b] == 0) part += s[b];
        S_U = block_sum<SIP_NT>(part, redf);
        int ncap = 0;
        for (int b = b0; b < b1; ++b)
          if (flag[b] == 0 && __fmul_rn(s[b], R) >= S_U) { flag[b] = 1; ++ncap; }
        ncap = block_sum_i<SIP_NT>(ncap, redi);
        if (ncap == 0) break;
        R -= (float)ncap;
        nfree -= ncap;
      }
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
    if (mode == 0) x = philox4x32_10({(uint32_t)(g >> 2), (uint32_t)i, (uint32_t)bh, ctr3}, key0, key1);
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
  int32_t* idx_row = kv_idx + (size_t)row * cap;
  float* w_row = inv_pi + (size_t)row * cap;
  for (int b = b0; b < b1; ++b) {
    if (flag[b] == 3) {
      idx_row[off] = b;
      w_row[off] = (mode == 0) ? __frcp_rn(s[b]) : 1.f;
      ++off;
    }
  }
  if (t == 0) count_out[row] = total;
}

// ============================================================================= launchers
hipError_t launch_select(const SelectLaunch& a, hipStream_t st) {
  const int BH = a.B * a.H;
  const int rows = BH * a.NQ;
  // K1
  {
    dim3 grid(a.NKp / 64, BH);
    if (a.d == 128)
      kv_block_mean_kernel<128><<<grid, 256, 0, st>>>(a.k, a.kbarT, a.L, a.Bk, a.NK, a.NKp);
    else
      kv_block_mean_kernel<64><<<grid, 256, 0, st>>>(a.k, a.kbarT, a.L, a.Bk, a.NK, a.NKp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // K2a
  {
    if (a.d == 128)
      ibcs_kmeans_kernel<128><<<rows, 256, 0, st>>>(a.q, a.mu, a.nj, a.L, a.Bq, a.NQ, a.C, a.Tk);
    else
      ibcs_kmeans_kernel<64><<<rows, 256, 0, st>>>(a.q, a.mu, a.nj, a.L, a.Bq, a.NQ, a.C, a.Tk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // K2b
  {
    const int rpw = 128 / a.C;
    dim3 grid((a.NQ + rpw - 1) / rpw, BH);
    const size_t lds = (size_t)a.d * (128 + 64) * sizeof(float);
#define ABSA_SCORE(DD, CC)                                                                         \
  ibcs_score_kernel<DD, CC><<<grid, 256, lds, st>>>(a.kbarT, a.mu, a.nj, a.s, a.L, a.Bk, a.Bq, a.NQ, \
                                                    a.NK, a.NKp, a.alpha)
    if (a.d == 128) {
      switch (a.C) {
        case 1: ABSA_SCORE(128, 1); break;
        case 2: ABSA_SCORE(128, 2); break;
        case 4: ABSA_SCORE(128, 4); break;
        default: ABSA_SCORE(128, 8); break;
      }
    } else {
      switch (a.C) {
        case 1: ABSA_SCORE(64, 1); break;
        case 2: ABSA_SCORE(64, 2); break;
        case 4: ABSA_SCORE(64, 4); break;
        default: ABSA_SCORE(64, 8); break;
      }
    }
#undef ABSA_SCORE
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // K3
  {
    const size_t lds = (size_t)a.NK * (sizeof(float) + 1);
    sip_kernel<<<rows, SIP_NT, lds, st>>>(a.s, a.NK, a.NQ, a.nstar, a.kstar, a.mode, a.key0, a.key1,
                                          a.ctr3, a.count, a.kv_idx, a.inv_pi, a.cap, a.pi_out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t configure_select_kernels() {
  // The scoring kernel uses 96 KB of dynamic LDS at d = 128.
  const int lds128 = 128 * (128 + 64) * (int)sizeof(float);
  hipError_t e;
#define ABSA_ATTR(DD, CC)                                                                  \
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ibcs_score_kernel<DD, CC>),      \
                          hipFuncAttributeMaxDynamicSharedMemorySize, lds128);             \
  if (e != hipSuccess) return e;
  ABSA_ATTR(128, 1) ABSA_ATTR(128, 2) ABSA_ATTR(128, 4) ABSA_ATTR(128, 8)
  ABSA_ATTR(64, 1) ABSA_ATTR(64, 2) ABSA_ATTR(64, 4) ABSA_ATTR(64, 8)
#undef ABSA_ATTR
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&sip_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, 12288 * 5);
  return e;
}

}  // namespace absa
