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
  {
    // 128 x D bf16 = 128 x D/8 16-byte chunks; every load is issued before any store
    constexpr int CH = D / 8, PER = 128 * CH / 256;
    const uint4* src = reinterpret_cast<const uint4*>(q + ((size_t)bh * L + q0) * D);
    uint4 wv[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int idx = t + 256 * j;
      wv[j] = (idx / CH < n) ? src[idx] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int idx = t + 256 * j;
      const int qq = idx / CH, cp = (idx % CH) * 4;
      if (qq < n) {
        X[qq * XS + cp + 0] = wv[j].x;
        X[qq * XS + cp + 1] = wv[j].y;
        X[qq * XS + cp + 2] = wv[j].z;
        X[qq * XS + cp + 3] = wv[j].w;
      }
    }
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
// Block logits l[row][j][b] = alpha * (mu_j . kbar_b) for every centroid of a
// head against every KV block: a [NQ*C x d] x [d x NK] product on fp32 MFMA
// (v_mfma_f32_32x32x2_f32, fp32 products and sums).  Workgroup = 4 waves x 32
// centroids; a wave keeps its centroids as A operands in registers and streams
// 32-block tiles of kbar^T through LDS.  Grid (ceil(M/128), BH, nsplit): split
// z covers a contiguous range of 32-block tiles.
template <int D>
__global__ __launch_bounds__(256) void ibcs_logit_kernel(const float* __restrict__ kbarT,
                                                         const float* __restrict__ mu,
                                                         float* __restrict__ logit, int M, int NK,
                                                         int NKp, int tiles_per_split, float alpha) {
  constexpr int KS = D / 2;  // k-steps of 2 dims
  __shared__ __attribute__((aligned(16))) float kt[2][D * 32];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int h = lane >> 5, n = lane & 31;
  const int bh = blockIdx.y;
  const int m0 = blockIdx.x * 128 + w * 32;
  const int tile0 = blockIdx.z * tiles_per_split;
  const int ntile_all = NKp / 32;
  const int tile1 = min(ntile_all, tile0 + tiles_per_split);
  if (tile0 >= tile1) return;

  // A operands: lane (h, n) holds mu[m0 + n][2 s + h]
  float areg[KS];
  {
    const int m = m0 + n;
    const float* src = mu + ((size_t)bh * M + (m < M ? m : 0)) * D;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) areg[s2] = (m < M) ? src[2 * s2 + h] : 0.f;
  }
  const float* kb = kbarT + (size_t)bh * D * NKp;
  float4 stage[D / 32];
  auto fetch = [&](int tile) {
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      const int idx = t + 256 * i;  // float4 index in the [D][32] tile
      const int c = idx >> 3, b4 = idx & 7;
      stage[i] = *reinterpret_cast<const float4*>(kb + (size_t)c * NKp + tile * 32 + b4 * 4);
    }
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      const int idx = t + 256 * i;
      *reinterpret_cast<float4*>(&kt[buf][idx * 4]) = stage[i];
    }
  };
  fetch(tile0);
  put(0);
  float* out_base = logit + (size_t)bh * M * NK;
#pragma unroll 1
  for (int tile = tile0; tile < tile1; ++tile) {
    const int buf = (tile - tile0) & 1;
    __syncthreads();
    if (tile + 1 < tile1) fetch(tile + 1);
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(areg[s2], kt[buf][(2 * s2 + h) * 32 + n], acc, 0, 0, 0);
    const int b = tile * 32 + n;
    if (b < NK) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (m < M) out_base[(size_t)m * NK + b] = alpha * acc[r];
      }
    }
    if (tile + 1 < tile1) put(buf ^ 1);
  }
}

// ============================================================================= K3
// One workgroup per row: inclusion probabilities by iterative capping, Philox
// Bernoulli draws (or top-k / all), and compaction into the row's list.
constexpr int SIP_NT = 256;

template <int C>
__global__ __launch_bounds__(SIP_NT) void sip_kernel(const float* __restrict__ logit,
                                                     const int* __restrict__ nj,
                                                     float* __restrict__ s_out, int L, int Bq, int Bk,
                                                     int NK, int NQ,
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
  __shared__ float redm[C][SIP_NT / 64], redz[C][SIP_NT / 64];
  const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
  const int row = blockIdx.x;
  const int bh = row / NQ, i = row % NQ;

  // ---- IBCS scores of this row from its logits: per centroid the max m_j and
  // the normaliser Z_j = sum_b nk_b 2^(l_jb - m_j) (terms below 2^-64 of the
  // max dropped), then s_b = sum_j (n_j/n) nk_b 2^(l_jb - m_j) / Z_j.
  {
    const float* lrow = logit + (size_t)row * C * NK;
    float mj[C], zj[C];
#pragma unroll
    for (int j = 0; j < C; ++j) { mj[j] = -INFINITY; zj[j] = 0.f; }
    constexpr int U = 4;  // blocks per batch: U*C loads in flight
#pragma unroll 1
    for (int b0 = t; b0 < NK; b0 += U * SIP_NT) {
      float lv[U][C];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < C; ++j) {
          const int b = b0 + u * SIP_NT;
          lv[u][j] = (b < NK) ? lrow[(size_t)j * NK + b] : -INFINITY;
        }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int b = b0 + u * SIP_NT;
        if (b >= NK) break;
        const float nk = (float)min(Bk, L - b * Bk);
#pragma unroll
        for (int j = 0; j < C; ++j) {
          const float l = lv[u][j];
          if (l > mj[j]) {
            zj[j] = (mj[j] - l >= -64.f) ? fmaf(zj[j], exp2_split(mj[j] - l), nk) : nk;
            mj[j] = l;
          } else if (l - mj[j] >= -64.f) {
            zj[j] = fmaf(nk, exp2_split(l - mj[j]), zj[j]);
          }
        }
      }
    }
    // combine (m, Z) pairs: lanes, then waves
#pragma unroll
    for (int j = 0; j < C; ++j) {
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float m2 = __shfl_xor(mj[j], o, 64), z2 = __shfl_xor(zj[j], o, 64);
        const float m = fmaxf(mj[j], m2);
        float z = 0.f;
        if (mj[j] - m >= -64.f) z += zj[j] * exp2_split(mj[j] - m);
        if (m2 - m >= -64.f) z += z2 * exp2_split(m2 - m);
        mj[j] = m;
        zj[j] = z;
      }
      if (lane == 0) { redm[j][wid] = mj[j]; redz[j][wid] = zj[j]; }
    }
    __syncthreads();
    const int n = min(Bq, L - i * Bq);
    float coef[C];
#pragma unroll
    for (int j = 0; j < C; ++j) {
      float m = -INFINITY;
#pragma unroll
      for (int w = 0; w < SIP_NT / 64; ++w) m = fmaxf(m, redm[j][w]);
      float z = 0.f;
#pragma unroll
      for (int w = 0; w < SIP_NT / 64; ++w)
        if (redm[j][w] - m >= -64.f) z += redz[j][w] * exp2_split(redm[j][w] - m);
      mj[j] = m;
      const int cnt = nj[(size_t)row * C + j];
      coef[j] = (cnt > 0) ? __fdiv_rn(__fdiv_rn((float)cnt, (float)n), z) : 0.f;
    }
    float* srow_out = s_out + (size_t)row * NK;
#pragma unroll 1
    for (int b0 = t; b0 < NK; b0 += U * SIP_NT) {
      float lv[U][C];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < C; ++j) {
          const int b = b0 + u * SIP_NT;
          lv[u][j] = (b < NK) ? lrow[(size_t)j * NK + b] : -INFINITY;
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
    const int M = a.NQ * a.C;
    const int mtiles = (M + 127) / 128;
    const int ntile_all = a.NKp / 32;
    int nsplit = (2048 + mtiles * BH - 1) / (mtiles * BH);
    nsplit = nsplit < 1 ? 1 : (nsplit > ntile_all ? ntile_all : nsplit);
    const int per = (ntile_all + nsplit - 1) / nsplit;
    nsplit = (ntile_all + per - 1) / per;
    dim3 grid(mtiles, BH, nsplit);
    if (a.d == 128)
      ibcs_logit_kernel<128><<<grid, 256, 0, st>>>(a.kbarT, a.mu, a.logit, M, a.NK, a.NKp, per, a.alpha);
    else
      ibcs_logit_kernel<64><<<grid, 256, 0, st>>>(a.kbarT, a.mu, a.logit, M, a.NK, a.NKp, per, a.alpha);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // K3
  {
    const size_t lds = (size_t)a.NK * (sizeof(float) + 1);
#define ABSA_SIP(CC)                                                                                  \
  sip_kernel<CC><<<rows, SIP_NT, lds, st>>>(a.logit, a.nj, a.s, a.L, a.Bq, a.Bk, a.NK, a.NQ, a.nstar,  \
                                            a.kstar, a.mode, a.key0, a.key1, a.ctr3, a.count, a.kv_idx, \
                                            a.inv_pi, a.cap, a.pi_out)
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
