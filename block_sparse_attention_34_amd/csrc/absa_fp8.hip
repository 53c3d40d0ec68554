// FP8 (E4M3) variant of the gather-attention step for gfx950 (VC-Attention
// page, section "İki darboğaz": value error dominates low-bit attention and a
// per-block mean of V removes part of it; softmax probabilities are written as
// E4M3 bytes directly by one fused multiply-add; section "Ölçümler": composes
// with sparse attention).  The quantisation and probability rules are listed in
// absa.h.  Fixed shape: d = 128, 128-query blocks, 16-key KV blocks.
//
// Pre-pass (three streaming kernels plus a per-head reduction):
//   fp8_q_kernel         per-token scale and codes of Q;
//   fp8_kv_stats_kernel  per 16-block chunk: fp64 column sums of K, the bf16
//                        block means of V and the chunk's max |v - mu_hat| per
//                        channel;
//   fp8_head_kernel      per head: kbar and the per-channel V scale;
//   fp8_kv_quant_kernel  K codes with per-block scales, V residual codes in the
//                        block-transposed layout, mu_hat / s_V as bf16 operands.
//
// Attention (attend_fp8_kernel) keeps the two-row anti-phase schedule of the
// bf16 kernel (absa_attend_pp.hip) and changes the tile arithmetic:
//   S^T = K Q^T and O^T += R^T P^T on v_mfma_f32_32x32x64_f8f6f4 (E4M3 both
//   operands; lane l holds k = 32 (l / 32) + byte of operand row / column
//   l % 32).  The key rows of the QK product are permuted so that lane (h, n)
//   ends up with all 16 keys of list entries 2h and 2h+1 for query n, which is
//   exactly the 32 consecutive keys its P operand must hold for the PV product.
//   The block sums S_b = sum_{k in b} p_k come from one more f8f6f4 product with
//   a 0/1 block-indicator operand; the mean term sum_b S_b mu_hat_b / s_V joins
//   O^T through one v_mfma_f32_32x32x16_bf16 per 32 channels, with S split into
//   bf16 high and low parts (both in one product: k = 0..3 carry the high
//   parts, k = 4..7 the low parts).  The per-channel scale s_V multiplies O at
//   the end.
//   With INT8 QK (codes clip(rne(x / s), -127, 127), s = 2^e for 127) the QK
//   product runs on v_mfma_i32_32x32x32_i8 instead (lane l holds k = 16 (l / 32)
//   + byte), whose int32 dot products are exact.
//   Logits: y = fma(acc, 8 scale log2(e) s_Q s_K, 8 (log2 w - m) + 120), one
//   fused multiply-add from the accumulator; P byte = v_cvt_pk_u8_f32(y)
//   (round to nearest even, clamped to [0, 255]).  The reference m is an
//   integer and y <= 120 after every rescale, so every byte is a finite E4M3
//   code and the rescale factors are exact powers of two.
#include <type_traits>

#include "absa_attend_tiles.h"
#include "absa_device.h"
#include "absa_launch.h"

namespace absa {

namespace {

constexpr int FD = 128;  // head dimension of the FP8 path
constexpr int FBK = 16;  // KV block size of the FP8 path

// exponent of the power-of-two scale: the smallest e with amax <= 448 * 2^e (0 for amax == 0)
__device__ __forceinline__ int pow2_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int k;
  const float m = frexpf(amax, &k);  // amax = m 2^k, m in [0.5, 1); 448 = 0.875 2^9
  return m <= 0.875f ? k - 9 : k - 8;
}

// INT8 QK: the smallest e with amax <= 127 * 2^e (0 for amax == 0)
__device__ __forceinline__ int pow2_exp_i8(float amax) {
  if (!(amax > 0.f)) return 0;
  int k;
  const float m = frexpf(amax, &k);  // 127 = 0.9921875 2^7
  return m <= 0.9921875f ? k - 7 : k - 6;
}

template <bool QI8>
__device__ __forceinline__ int qk_exp(float amax) {
  return QI8 ? pow2_exp_i8(amax) : pow2_exp(amax);
}

__device__ __forceinline__ void unpack8(const u32x4 w, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// E4M3 codes (round to nearest even) of x[0..3] * 2^-e, packed little-endian
__device__ __forceinline__ uint32_t codes4(float x0, float x1, float x2, float x3, int e) {
  const float a0 = ldexpf(x0, -e), a1 = ldexpf(x1, -e), a2 = ldexpf(x2, -e), a3 = ldexpf(x3, -e);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, w, true);
  return (uint32_t)w;
}

// INT8 codes clip(rne(x * 2^-e), -127, 127) of x[0..3], packed little-endian
__device__ __forceinline__ uint32_t codes4_i8(float x0, float x1, float x2, float x3, int e) {
  const float xs[4] = {x0, x1, x2, x3};
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float r = fminf(fmaxf(rintf(ldexpf(xs[i], -e)), -127.f), 127.f);
    w |= ((uint32_t)(int)r & 0xFFu) << (8 * i);
  }
  return w;
}

template <bool QI8>
__device__ __forceinline__ uint32_t qk_codes4(float x0, float x1, float x2, float x3, int e) {
  return QI8 ? codes4_i8(x0, x1, x2, x3, e) : codes4(x0, x1, x2, x3, e);
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {  // round to nearest even
  const __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

}  // namespace

// ============================================================================= pre-pass
// grid (ceil(L/16), BH), 256 threads: 16 tokens per workgroup, 16 lanes per token
template <bool QI8>
__global__ __launch_bounds__(256) void fp8_q_kernel(const uint16_t* __restrict__ q, uint8_t* __restrict__ q8,
                                                    float* __restrict__ sq, int L) {
  const int t = threadIdx.x, cl = t & 15;
  const int tok = blockIdx.x * 16 + (t >> 4);
  const size_t bh = blockIdx.y;
  const bool ok = tok < L;
  const size_t row = bh * L + (ok ? tok : 0);
  u32x4 w = ok ? *reinterpret_cast<const u32x4*>(q + row * FD + 8 * cl) : u32x4{0u, 0u, 0u, 0u};
  float x[8];
  unpack8(w, x);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  const int e = qk_exp<QI8>(amax);
  if (ok) {
    const uint32_t c0 = qk_codes4<QI8>(x[0], x[1], x[2], x[3], e), c1 = qk_codes4<QI8>(x[4], x[5], x[6], x[7], e);
    *reinterpret_cast<uint2*>(q8 + row * FD + 8 * cl) = make_uint2(c0, c1);
    if (cl == 0) sq[row] = ldexpf(1.f, e);
  }
}

// grid (nchunk = ceil(NK/16), BH), 256 threads; thread (b = t/16, cl = t%16)
// covers block 16 chunk + b, channels 8 cl .. 8 cl + 7.
//   ksum_part [BH][nchunk][128] fp64   column sums of K over the chunk's tokens
//   vmax_part [BH][nchunk][128] fp32   max |v - mu_hat| over the chunk's tokens
//   mu_nat    [BH][NK][128] bf16       block means mu_hat
__global__ __launch_bounds__(256) void fp8_kv_stats_kernel(const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ v,
                                                           double* __restrict__ ksum_part,
                                                           float* __restrict__ vmax_part,
                                                           uint16_t* __restrict__ mu_nat, int L, int NK) {
  __shared__ double ks[16][FD];
  __shared__ float vm[16][FD];
  const int t = threadIdx.x, b = t >> 4, cl = t & 15;
  const size_t bh = blockIdx.y;
  const int nchunk = gridDim.x;
  const int blk = blockIdx.x * 16 + b;
  const int t0 = blk * FBK;
  const int n = blk < NK ? min(FBK, L - t0) : 0;
  double kacc[8], vacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) kacc[i] = vacc[i] = 0.0;
  u32x4 vw[FBK];
#pragma unroll
  for (int j = 0; j < FBK; ++j) {
    const bool ok = j < n;
    const size_t off = (bh * L + (ok ? t0 + j : 0)) * FD + 8 * cl;
    const u32x4 kw = ok ? *reinterpret_cast<const u32x4*>(k + off) : u32x4{0u, 0u, 0u, 0u};
    vw[j] = ok ? *reinterpret_cast<const u32x4*>(v + off) : u32x4{0u, 0u, 0u, 0u};
    float xk[8], xv[8];
    unpack8(kw, xk);
    unpack8(vw[j], xv);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      kacc[i] += (double)xk[i];
      vacc[i] += (double)xv[i];
    }
  }
  float muh[8];
  float amax[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    muh[i] = n > 0 ? (float)(vacc[i] / (double)n) : 0.f;
    muh[i] = __uint_as_float((uint32_t)bf16_bits(muh[i]) << 16);
    amax[i] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < FBK; ++j) {
    if (j < n) {
      float xv[8];
      unpack8(vw[j], xv);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax[i] = fmaxf(amax[i], fabsf(xv[i] - muh[i]));
    }
  }
  if (n > 0) {
    u32x4 mw;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      mw[i] = (uint32_t)bf16_bits(muh[2 * i]) | ((uint32_t)bf16_bits(muh[2 * i + 1]) << 16);
    *reinterpret_cast<u32x4*>(mu_nat + (bh * NK + blk) * FD + 8 * cl) = mw;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    ks[b][8 * cl + i] = kacc[i];
    vm[b][8 * cl + i] = amax[i];
  }
  __syncthreads();
  if (t < FD) {
    double s = 0.0;
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      s += ks[j][t];
      m = fmaxf(m, vm[j][t]);
    }
    ksum_part[(bh * nchunk + blockIdx.x) * FD + t] = s;
    vmax_part[(bh * nchunk + blockIdx.x) * FD + t] = m;
  }
}

// grid BH, 128 threads (one per channel)
__global__ __launch_bounds__(128) void fp8_head_kernel(const double* __restrict__ ksum_part,
                                                       const float* __restrict__ vmax_part, float* __restrict__ kbar,
                                                       float* __restrict__ sv, int nchunk, int L) {
  const int c = threadIdx.x;
  const size_t bh = blockIdx.x;
  double s = 0.0;
  float m = 0.f;
  for (int j = 0; j < nchunk; ++j) {
    s += ksum_part[(bh * nchunk + j) * FD + c];
    m = fmaxf(m, vmax_part[(bh * nchunk + j) * FD + c]);
  }
  kbar[bh * FD + c] = (float)(s / (double)L);
  sv[bh * FD + c] = ldexpf(1.f, pow2_exp(m));
}

// grid (nchunk, BH), 256 threads; thread (b = t/16, cl = t%16) as in the stats kernel
template <bool QI8>
__global__ __launch_bounds__(256) void fp8_kv_quant_kernel(const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ v,
                                                           const uint16_t* __restrict__ mu_nat,
                                                           const float* __restrict__ kbar,
                                                           const float* __restrict__ sv, uint8_t* __restrict__ k8,
                                                           float* __restrict__ sk, uint8_t* __restrict__ v8t,
                                                           uint16_t* __restrict__ mu_op, int L, int NK) {
  const int t = threadIdx.x, b = t >> 4, cl = t & 15;
  const size_t bh = blockIdx.y;
  const int blk = blockIdx.x * 16 + b;
  const bool bok = blk < NK;
  const int t0 = blk * FBK;
  const int n = bok ? min(FBK, L - t0) : 0;
  float kb[8], ev[8], muh[8];
  {
    const float4 k0 = *reinterpret_cast<const float4*>(kbar + bh * FD + 8 * cl);
    const float4 k1 = *reinterpret_cast<const float4*>(kbar + bh * FD + 8 * cl + 4);
    kb[0] = k0.x; kb[1] = k0.y; kb[2] = k0.z; kb[3] = k0.w;
    kb[4] = k1.x; kb[5] = k1.y; kb[6] = k1.z; kb[7] = k1.w;
    const float4 s0 = *reinterpret_cast<const float4*>(sv + bh * FD + 8 * cl);
    const float4 s1 = *reinterpret_cast<const float4*>(sv + bh * FD + 8 * cl + 4);
    const float sv8[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int e;
      frexpf(sv8[i], &e);
      ev[i] = (float)(e - 1);  // sv = 2^(e-1)
    }
    u32x4 mw = bok ? *reinterpret_cast<const u32x4*>(mu_nat + (bh * NK + (bok ? blk : 0)) * FD + 8 * cl)
                   : u32x4{0u, 0u, 0u, 0u};
    unpack8(mw, muh);
  }
  // ---- K: k - kbar, block max, codes
  float kc[FBK][8];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < FBK; ++j) {
    const bool ok = j < n;
    const size_t off = (bh * L + (ok ? t0 + j : 0)) * FD + 8 * cl;
    const u32x4 kw = ok ? *reinterpret_cast<const u32x4*>(k + off) : u32x4{0u, 0u, 0u, 0u};
    float xk[8];
    unpack8(kw, xk);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      kc[j][i] = ok ? xk[i] - kb[i] : 0.f;
      amax = fmaxf(amax, fabsf(kc[j][i]));
    }
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  const int ek = qk_exp<QI8>(amax);
#pragma unroll
  for (int j = 0; j < FBK; ++j) {
    if (j < n) {
      const uint32_t c0 = qk_codes4<QI8>(kc[j][0], kc[j][1], kc[j][2], kc[j][3], ek);
      const uint32_t c1 = qk_codes4<QI8>(kc[j][4], kc[j][5], kc[j][6], kc[j][7], ek);
      *reinterpret_cast<uint2*>(k8 + (bh * L + t0 + j) * FD + 8 * cl) = make_uint2(c0, c1);
    }
  }
  if (bok && cl == 0) sk[bh * NK + blk] = ldexpf(1.f, ek);
  if (!bok) return;
  // ---- V: residual codes, 16 keys of a channel contiguous
  float rv[FBK][8];
#pragma unroll
  for (int j = 0; j < FBK; ++j) {
    const bool ok = j < n;
    const size_t off = (bh * L + (ok ? t0 + j : 0)) * FD + 8 * cl;
    const u32x4 vw = ok ? *reinterpret_cast<const u32x4*>(v + off) : u32x4{0u, 0u, 0u, 0u};
    float xv[8];
    unpack8(vw, xv);
#pragma unroll
    for (int i = 0; i < 8; ++i) rv[j][i] = ok ? xv[i] - muh[i] : 0.f;
  }
  uint8_t* vrow = v8t + (bh * NK + blk) * (size_t)(FD * FBK);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = (int)ev[i];
    u32x4 w;
#pragma unroll
    for (int g = 0; g < 4; ++g) w[g] = codes4(rv[4 * g][i], rv[4 * g + 1][i], rv[4 * g + 2][i], rv[4 * g + 3][i], e);
    *reinterpret_cast<u32x4*>(vrow + (8 * cl + i) * FBK) = w;
    // mu_hat / s_V (exact: a power-of-two scaling of a bf16 value) in the operand order
    const int c = 8 * cl + i;
    mu_op[(bh * NK + blk) * FD + (c & 31) * 4 + (c >> 5)] = bf16_bits(ldexpf(muh[i], -e));
  }
}

// ============================================================================= attention
template <bool DENSE, bool OUT_BF16, bool QI8>
__global__ __launch_bounds__(512, 1) void attend_fp8_kernel(AttendFp8Launch a) {
  constexpr int D = FD, BK = FBK, BQ = 128;
  constexpr int NW = 4;              // waves per row, 32 queries each
  constexpr int SPT = 64 / BK;       // list entries per 64-key tile (4)
  constexpr int NCH = 2;             // 1 KB wave-wide loads per wave, tile and tensor
  constexpr int KT = 64 * D;         // K tile bytes (8 KB)
  constexpr int VT = SPT * D * BK;   // V tile bytes (8 KB)
  constexpr int MT = SPT * 256;      // block-mean operands of a tile (1 KB)
  typedef int v8i __attribute__((ext_vector_type(8)));
  typedef int v4i __attribute__((ext_vector_type(4)));
  typedef int v16i __attribute__((ext_vector_type(16)));

  constexpr int ST = 4 * 256;        // s_K of a tile: each wave lands 64 lanes x 4 B, wave 0's is read
  // one LDS object per slot, the loop unrolled by two: every slot a phase
  // touches is a compile-time constant, so the compiler sees that a phase's LDS
  // reads never alias the direct loads in flight into the other slots  [row][bytes]
  __shared__ __attribute__((aligned(16))) unsigned char k_s0[2][KT + ST], k_s1[2][KT + ST];
  __shared__ __attribute__((aligned(16))) unsigned char v_s0[2][VT + MT], v_s1[2][VT + MT];

  const int npairs = (a.rows + 1) >> 1;
  int pair = blockIdx.x;
  {
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
      nb = a.NK;
      return (a.NK + SPT - 1) / SPT;
    } else {
      int c = a.count[r];
      c = c < 0 ? 0 : (c > a.cap ? a.cap : c);
      nb = c;
      return (c + SPT - 1) / SPT;
    }
  };
  const int row = 2 * pair + half, orow = 2 * pair + (1 - half);
  int nblk = 0, onb = 0;
  const int T = row < a.rows ? list_len(row, nblk) : 0;
  const int To = orow < a.rows ? list_len(orow, onb) : 0;
  const int rowc = row < a.rows ? row : a.rows - 1;
  const int bh = rowc / a.NQ, qb = rowc % a.NQ;
  const size_t head_tok = (size_t)bh * a.L;
  const int qi = qb * BQ + wq * 32 + qn;
  const bool qvalid = row < a.rows && qi < a.L;

  if (row < a.rows && T == 0 && qvalid) {  // empty list: the estimate is 0
#pragma unroll
    for (int c = 0; c < D; c += 4) {
      if constexpr (OUT_BF16)
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.o) + (head_tok + qi) * D + c) = make_uint2(0, 0);
      else
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.o) + (head_tok + qi) * D + c) =
            make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }

  // ---- this lane's query as the B operand of S^T = K Q^T: E4M3, two k-steps of
  // 64 (bytes 64 ks + 32 h ..); INT8, four k-steps of 32 (bytes 32 ks + 16 h ..).
  // qw[i] is the 16-byte chunk i of the lane's 64 operand bytes.
  u32x4 qw[4];
  float qs8;  // 8 scale log2(e) s_Q of this query
  {
    const u32x4* qp = reinterpret_cast<const u32x4*>(a.q8 + (head_tok + (qvalid ? qi : 0)) * D);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = QI8 ? 2 * i + h : 4 * (i >> 1) + 2 * h + (i & 1);
      qw[i] = qvalid ? qp[c] : u32x4{0u, 0u, 0u, 0u};
    }
    qs8 = 8.f * a.scale_log2 * (qvalid ? a.sq[head_tok + qi] : 1.f);
  }
  const int32_t* lidx = DENSE ? nullptr : a.kv_idx + (size_t)rowc * a.cap;
  const float* lw = DENSE ? nullptr : a.inv_pi + (size_t)rowc * a.cap;

  // ---- direct loads: K codes [L][128] (an entry's 16 rows are 2 KB), V codes
  // [NK][128][16] (2 KB per block) and the block-mean operands [NK][256 B];
  // invalid entries get a base past the resources, so their loads land zeros.
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.k8 + head_tok * D), 0, (int)((uint32_t)a.L * D), 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.v8t + (size_t)bh * a.NK * (D * BK)), 0, (int)((uint32_t)a.NK * D * BK), 0x00020000);
  const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.mu + (size_t)bh * a.NK * D), 0, (int)((uint32_t)a.NK * D * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t srs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.sk + (size_t)bh * a.NK), 0, (int)((uint32_t)a.NK * 4), 0x00020000);
  constexpr uint32_t OOB = 0x7FFFFFF0u;
  // K tile in LDS: row r (tile key r), 16-byte chunk c stored at chunk c ^ ks(r);
  // wave-wide load j of wave wq fills rows 8 ci .. 8 ci + 7, ci = j NW + wq
  auto kswz = [](int r) { return ((r >> 1) & 3) | ((r >> 3) & 4); };
  uint32_t klane[NCH], vlane[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int ci = j * NW + wq;
    const int r = 8 * ci + (lane >> 3), pc = lane & 7;
    klane[j] = (uint32_t)((r & 15) * D + ((pc ^ kswz(r)) << 4));
    vlane[j] = (uint32_t)((64 * (ci & 1) + lane) * 16);  // V block ci/2, channel rows 64 (ci&1) + lane
  }
  const uint32_t mlane = (uint32_t)lane * 4;  // wave wq loads the 256 B operand record of entry wq

  struct Entry {
    int blk;
    float w;
  };
  auto fetch = [&](Entry& E, int tile) {
    const int e = tile * SPT + lane % SPT;
    if constexpr (DENSE) {
      E.blk = e;
      E.w = 1.f;
    } else {
      const int last = nblk > 0 ? nblk - 1 : 0;
      const int ec = e < last ? e : last;
      E.blk = lidx[ec];
      E.w = lw[ec];
    }
  };
  // decoded tile: per lane (entry lane % SPT) the bias log2 w (-inf outside the
  // list) and the mask of keys past L; per wave the byte bases of its K/V loads
  // and of its block-mean load, per lane the offset of its entry's s_K (the
  // scales travel with the K tile into LDS, so no register ever waits on them)
  struct Tile {
    float bias;
    unsigned long long past;
  };
  struct Bases {
    uint32_t kv[NCH];
    uint32_t mu;
    uint32_t sk;
  };
  auto decode = [&](const Entry& E, int tile, Bases& bs, Tile& t) {
    const int e = tile * SPT + lane % SPT;
    const bool ok = e < nblk && (unsigned)E.blk < (unsigned)a.NK;
    const uint32_t bb = ok ? (uint32_t)E.blk * (D * BK) : OOB;
    const uint32_t mb = ok ? (uint32_t)E.blk * (D * 2) : OOB;
#pragma unroll
    for (int j = 0; j < NCH; ++j) bs.kv[j] = __builtin_amdgcn_readlane(bb, (j * NW + wq) >> 1);
    bs.mu = __builtin_amdgcn_readlane(mb, wq);
    bs.sk = ok ? (uint32_t)E.blk * 4 : OOB;
    t.bias = ok ? (DENSE ? 0.f : __log2f(E.w)) : -INFINITY;
    t.past = 0ull;
    if (__ballot(ok && (E.blk + 1) * BK > a.L) != 0ull) {  // the block holding key L-1
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
  };
  auto dma = [&](const Bases& bs, unsigned char* kbuf, unsigned char* vbuf, bool do_k, bool do_v) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int ci = j * NW + wq;
      if (do_k) {
        const int off = (int)(klane[j] + bs.kv[j]);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void_t*)(kbuf + ci * 1024), 16, off, 0, 0, 0);
      }
      if (do_v) {
        const int off = (int)(vlane[j] + bs.kv[j]);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void_t*)(vbuf + ci * 1024), 16, off, 0, 0, 0);
      }
    }
    if (do_k) {
      const int off = (int)bs.sk;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (lds_void_t*)(kbuf + KT + wq * 256), 4, off, 0, 0, 0);
    }
    if (do_v) {
      const int off = (int)(mlane + bs.mu);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(mrs, (lds_void_t*)(vbuf + VT + wq * 256), 4, off, 0, 0, 0);
    }
  };

  // ---- per-lane LDS read offsets.  QK row i of key half sb holds tile key
  // 32 ((i >> 2) & 1) + 16 sb + 4 (i >> 3) + (i & 3), so that accumulator
  // element r of lane (h, n) in half sb is key 32 h + 16 sb + r.
  int koff[4];  // the four 16-byte chunks of this lane's K operand bytes (as qw), sb = 0; sb = 1 adds 16 rows
  {
    const int i = qn;
    const int r = 32 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = QI8 ? 2 * j + h : 4 * (j >> 1) + 2 * h + (j & 1);
      koff[j] = r * D + ((c ^ kswz(r)) << 4);
    }
  }
  // PV A operand (R^T): lane (h, c) reads channel row 32 cb + c of entries 2h, 2h+1
  const int voff = (2 * h) * (D * BK) + qn * 16;
  // E operand: row i of the block indicator, k = 32 h + byte
  v8i eop;
  {
    const int on = 0x38383838;  // four E4M3 ones
#pragma unroll
    for (int d8 = 0; d8 < 8; ++d8) eop[d8] = ((qn == 2 * h && d8 < 4) || (qn == 2 * h + 1 && d8 >= 4)) ? on : 0;
  }

  f32x16 acc[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;
  f32x16 sacc[2];
  v8i pf;  // P bytes of the current tile: byte 16 sb + r = key 32 h + 16 sb + r
  float m_run = -INFINITY, l_run = 0.f;

  // S^T = K Q^T; with INT8 the exact int32 dot products (|acc| <= 127^2 128 < 2^24)
  // are converted to fp32 exactly
  auto qk = [&](const unsigned char* kb) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[sb][r] = 0.f;
    if constexpr (QI8) {
      v16i iacc[2] = {};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          const u32x4 x = *reinterpret_cast<const u32x4*>(kb + koff[ks] + sb * 16 * D);
          const v4i kfrag = {(int)x[0], (int)x[1], (int)x[2], (int)x[3]};
          const v4i qfrag = {(int)qw[ks][0], (int)qw[ks][1], (int)qw[ks][2], (int)qw[ks][3]};
          iacc[sb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kfrag, qfrag, iacc[sb], 0, 0, 0);
        }
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[sb][r] = (float)iacc[sb][r];
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          const u32x4 x0 = *reinterpret_cast<const u32x4*>(kb + koff[2 * ks] + sb * 16 * D);
          const u32x4 x1 = *reinterpret_cast<const u32x4*>(kb + koff[2 * ks + 1] + sb * 16 * D);
          const v8i kfrag = {(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                             (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
          const v8i qfrag = {(int)qw[2 * ks][0], (int)qw[2 * ks][1], (int)qw[2 * ks][2], (int)qw[2 * ks][3],
                             (int)qw[2 * ks + 1][0], (int)qw[2 * ks + 1][1], (int)qw[2 * ks + 1][2],
                             (int)qw[2 * ks + 1][3]};
          sacc[sb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kfrag, qfrag, sacc[sb], 0, 0, 0, 0, 0, 0);
        }
    }
  };
  // O^T += R^T P^T (residual codes) and the block-mean term
  auto pv = [&](const unsigned char* vb) {
    const f32x16 zero = {};
    const f32x16 es = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(eop, pf, zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const u32x4 x0 = *reinterpret_cast<const u32x4*>(vb + voff + cb * 512);
      const u32x4 x1 = *reinterpret_cast<const u32x4*>(vb + voff + D * BK + cb * 512);
      const v8i vfrag = {(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
      acc[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vfrag, pf, acc[cb], 0, 0, 0, 0, 0, 0);
    }
    // block sums S_b (rows 0..3 of es live in lanes h = 0; lanes h = 1 hold zeros)
    uint32_t sw[4];
    float srow = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float s0 = es[2 * i], s1 = es[2 * i + 1];
      const uint16_t h0 = bf16_bits(s0), h1 = bf16_bits(s1);
      const float r0 = s0 - __uint_as_float((uint32_t)h0 << 16), r1 = s1 - __uint_as_float((uint32_t)h1 << 16);
      sw[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
      sw[2 + i] = (uint32_t)bf16_bits(r0) | ((uint32_t)bf16_bits(r1) << 16);
      srow += s0 + s1;
    }
    l_run += srow;
    const bf16x8 sop = __builtin_bit_cast(bf16x8, u32x4{sw[0], sw[1], sw[2], sw[3]});
    // block-mean operands: entry e's record holds, at lane position c, the four
    // 32-channel groups of channel c + 32 j (bf16 pairs)
    uint2 mrec[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) mrec[e] = *reinterpret_cast<const uint2*>(vb + VT + e * 256 + qn * 8);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int sel = (cb & 1) ? 0x07060302 : 0x05040100;
      const uint32_t d01 = __builtin_amdgcn_perm((cb < 2) ? mrec[1].x : mrec[1].y, (cb < 2) ? mrec[0].x : mrec[0].y, sel);
      const uint32_t d23 = __builtin_amdgcn_perm((cb < 2) ? mrec[3].x : mrec[3].y, (cb < 2) ? mrec[2].x : mrec[2].y, sel);
      const bf16x8 mop = __builtin_bit_cast(bf16x8, u32x4{d01, d23, d01, d23});
      acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mop, sop, acc[cb], 0, 0, 0);
    }
  };

  // ---- vector work.  y = 8 (l - m_use) + 120 from the accumulators; element
  // r of half sb belongs to entry 2h + sb; returns this lane's max
  auto logits = [&](const Tile& tl, const unsigned char* kb, float m_use) {
    float bi[SPT];
#pragma unroll
    for (int i = 0; i < SPT; ++i)
      bi[i] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tl.bias), i));
    const float4 s4 = *reinterpret_cast<const float4*>(kb + KT);  // s_K of entries 0..3
    const float si[SPT] = {s4.x, s4.y, s4.z, s4.w};
    float mt = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const float bias = h ? bi[2 + sb] : bi[sb];
      const float skb = h ? si[2 + sb] : si[sb];
      const float mul = qs8 * skb;
      const float add = fmaf(bias - m_use, 8.f, 120.f);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float y = fmaf(sacc[sb][r], mul, add);
        sacc[sb][r] = y;
        mt = fmaxf(mt, y);
      }
    }
    return mt;
  };
  auto mask_tail = [&](const Tile& tl) {
    float mt = -INFINITY;
    const uint32_t w = (uint32_t)(tl.past >> (32 * h));
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if ((w >> (16 * sb + r)) & 1u) sacc[sb][r] = -INFINITY;
        mt = fmaxf(mt, sacc[sb][r]);
      }
    return mt;
  };
  // raise the integer reference when the tile holds a y above 120 (or on the
  // first tile with a finite logit) by the fewest whole octaves that bring the
  // tile's max to 120 or below: y -= 8 step, O and l scale by 2^-step.  The
  // reference so reached is the smallest integer that keeps every y of the row
  // at or below 120, whatever the order of the tiles; a term computed under an
  // earlier, lower reference keeps its byte's value exactly after the rescale
  // unless that byte falls below the normal range under the final one.
  auto rescale = [&](float mt, float m_use) {
    mt = half_swap_max(mt);
    const bool need = mt > 120.f || (m_run == -INFINITY && mt > -INFINITY);
    if (__ballot(need) != 0ull) {
      const float step = need ? ceilf((mt - 120.f) * 0.125f) : 0.f;
      const float alpha = need ? ((m_run == -INFINITY) ? 0.f : ldexpf(1.f, -(int)step)) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[cb][r] *= alpha;
      m_run = need ? m_use + step : m_run;
      const float sh8 = 8.f * step;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[sb][r] -= sh8;
    }
  };

  // ---- pipeline state (as in the bf16 two-row kernel): entering vector(m),
  // sacc holds y of tile m and mt its lane max; t1, t2 are tiles m+1, m+2;
  // kn the bases of tile m+2 (K) and vb of tile m+1 (V and block means)
  Entry EN;
  Bases kn, vb;
  Tile t1, t2, t3;
  float mt;
  auto form_logits = [&](const Tile& tl, const unsigned char* kb) {
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float x = logits(tl, kb, m_use);
    if (tl.past != 0ull) x = mask_tail(tl);
    return x;
  };
  {
    Entry E0, E1, E2;
    fetch(E0, 0);
    fetch(E1, 1);
    fetch(E2, 2);
    fetch(EN, 3);
    Bases b0;
    Tile t0;
    decode(E0, 0, b0, t0);
    dma(b0, K0, V0, true, true);
    decode(E1, 1, vb, t1);
    dma(vb, K1, nullptr, true, false);
    decode(E2, 2, kn, t2);
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    __syncthreads();
    qk(K0);
    mt = form_logits(t0, K0);
  }
  // one direct load of a vector phase, in dma()'s order: the K chunks, s_K, the
  // V chunks, the block means
  auto dma_one = [&](int i, unsigned char* kbuf, unsigned char* vbuf) {
    if (i < NCH) {
      const int off = (int)(klane[i] + kn.kv[i]);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void_t*)(kbuf + (i * NW + wq) * 1024), 16, off, 0, 0, 0);
    } else if (i == NCH) {
      const int off = (int)kn.sk;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (lds_void_t*)(kbuf + KT + wq * 256), 4, off, 0, 0, 0);
    } else if (i < 2 * NCH + 1) {
      const int j = i - NCH - 1;
      const int off = (int)(vlane[j] + vb.kv[j]);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void_t*)(vbuf + (j * NW + wq) * 1024), 16, off, 0, 0, 0);
    } else {
      const int off = (int)(mlane + vb.mu);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(mrs, (lds_void_t*)(vbuf + VT + wq * 256), 4, off, 0, 0, 0);
    }
  };
  // ExpCast: byte = sat_u8(rne(y)), four per dword.  Over gathered lists the
  // phase's 2 NCH + 2 direct loads go out one after each of the first dwords, so
  // that the CU's shared address unit works through them while the waves convert
  // (as one block the compiler issues them ahead of the conversions, and each
  // wave then stalls behind the queue); the empty statements keep the dwords in
  // this order.  Dense tiles hit in L2 and keep the block.
  auto probs_dma = [&](unsigned char* kbuf, unsigned char* vbuf) {
#pragma unroll
    for (int dw = 0; dw < 8; ++dw) {
      const int sb = dw >> 2, r0 = 4 * (dw & 3);
      uint32_t w = __builtin_amdgcn_cvt_pk_u8_f32(sacc[sb][r0], 0, 0u);
      w = __builtin_amdgcn_cvt_pk_u8_f32(sacc[sb][r0 + 1], 1, w);
      w = __builtin_amdgcn_cvt_pk_u8_f32(sacc[sb][r0 + 2], 2, w);
      w = __builtin_amdgcn_cvt_pk_u8_f32(sacc[sb][r0 + 3], 3, w);
      pf[dw] = (int)w;
      if constexpr (!DENSE) {
        asm volatile("" ::"v"(w));
        if (dw < 2 * NCH + 2) {
          dma_one(dw, kbuf, vbuf);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if constexpr (DENSE)
#pragma unroll
      for (int i = 0; i < 2 * NCH + 2; ++i) dma_one(i, kbuf, vbuf);
  };
  // loads issued by one vector phase: K (NCH) and V (NCH) direct loads, the
  // s_K and block-mean loads, and (lists) two entry loads
  constexpr int NLD = 2 * NCH + 2 + (DENSE ? 0 : 2);
  // (pc: the parity of m as a compile-time constant, which names the slots)
  auto vector_phase = [&](auto pc, int m) {
    constexpr int p = decltype(pc)::value;
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    rescale(mt, m_use);
    probs_dma(p ? K1 : K0, p ? V0 : V1);  // K(m+2), V(m+1) and its block means
    vb = kn;
    decode(EN, m + 3, kn, t3);
    fetch(EN, m + 4);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(NLD | 0x0070);  // vmcnt(NLD) lgkmcnt(0)
  };
  auto matrix_phase = [&](auto pc) {
    constexpr int p = decltype(pc)::value;
    qk(p ? K0 : K1);
    pv(p ? V1 : V0);
    mt = form_logits(t1, p ? K0 : K1);
    t1 = t2;
    t2 = t3;
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  };
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
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

  // ---- epilogue: O = s_V O^T / l, valid queries only
  if (T > 0) {
    const float l_tot = half_swap_sum(l_run);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    if (qvalid) {
      const size_t obase = (head_tok + qi) * D;
      const float* svh = a.sv + (size_t)bh * D;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int dc = cb * 32 + 8 * g4 + 4 * h;
          const float4 s = *reinterpret_cast<const float4*>(svh + dc);
          const float o0 = acc[cb][4 * g4 + 0] * s.x * inv, o1 = acc[cb][4 * g4 + 1] * s.y * inv;
          const float o2 = acc[cb][4 * g4 + 2] * s.z * inv, o3 = acc[cb][4 * g4 + 3] * s.w * inv;
          if constexpr (OUT_BF16) {
            const uint32_t w0 = (uint32_t)bf16_bits(o0) | ((uint32_t)bf16_bits(o1) << 16);
            const uint32_t w1 = (uint32_t)bf16_bits(o2) | ((uint32_t)bf16_bits(o3) << 16);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.o) + obase + dc) = make_uint2(w0, w1);
          } else {
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.o) + obase + dc) = make_float4(o0, o1, o2, o3);
          }
        }
    }
  }
}

// ============================================================================= launchers
hipError_t launch_quantize_fp8(const QuantFp8Launch& a, hipStream_t st) {
  const int nchunk = (a.NK + 15) / 16;
  if (a.qk_int8) fp8_q_kernel<true><<<dim3((a.L + 15) / 16, a.BH), 256, 0, st>>>(a.q, a.q8, a.sq, a.L);
  else fp8_q_kernel<false><<<dim3((a.L + 15) / 16, a.BH), 256, 0, st>>>(a.q, a.q8, a.sq, a.L);
  fp8_kv_stats_kernel<<<dim3(nchunk, a.BH), 256, 0, st>>>(a.k, a.v, a.ksum_part, a.vmax_part, a.mu_nat, a.L,
                                                           a.NK);
  fp8_head_kernel<<<dim3(a.BH), 128, 0, st>>>(a.ksum_part, a.vmax_part, a.kbar, a.sv, nchunk, a.L);
  if (a.qk_int8)
    fp8_kv_quant_kernel<true><<<dim3(nchunk, a.BH), 256, 0, st>>>(a.k, a.v, a.mu_nat, a.kbar, a.sv, a.k8, a.sk,
                                                                   a.v8t, a.mu, a.L, a.NK);
  else
    fp8_kv_quant_kernel<false><<<dim3(nchunk, a.BH), 256, 0, st>>>(a.k, a.v, a.mu_nat, a.kbar, a.sv, a.k8, a.sk,
                                                                    a.v8t, a.mu, a.L, a.NK);
  return hipGetLastError();
}

template <bool QI8>
static void launch_attend_fp8_t(const AttendFp8Launch& a, hipStream_t st, bool dense) {
  dim3 grid((a.rows + 1) / 2);
  if (dense) {
    if (a.out_bf16) attend_fp8_kernel<true, true, QI8><<<grid, 512, 0, st>>>(a);
    else attend_fp8_kernel<true, false, QI8><<<grid, 512, 0, st>>>(a);
  } else {
    if (a.out_bf16) attend_fp8_kernel<false, true, QI8><<<grid, 512, 0, st>>>(a);
    else attend_fp8_kernel<false, false, QI8><<<grid, 512, 0, st>>>(a);
  }
}

hipError_t launch_attend_fp8(const AttendFp8Launch& a, hipStream_t st, bool dense) {
  if (a.qk_int8) launch_attend_fp8_t<true>(a, st, dense);
  else launch_attend_fp8_t<false>(a, st, dense);
  return hipGetLastError();
}

}  // namespace absa
