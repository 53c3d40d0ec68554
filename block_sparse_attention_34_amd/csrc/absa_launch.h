// Launch descriptors passed from the C-ABI layer to the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace absa {

struct SelectLaunch {
  const uint16_t* q;
  const uint16_t* k;
  int B, H, L, d, Bq, Bk, NQ, NK, NKp, C, Tk, mode, kstar, cap;
  float nstar, alpha;
  uint32_t key0, key1, ctr3;
  float* kbarT;  // workspace: [BH][d][NKp], written only when not null
  uint16_t* kbh; // workspace: block means' bf16 heads and tails in matrix operand order
  float* mu;     // workspace: [rows][C][d]
  int* nj;       // workspace: [rows][C]
  float* s;      // workspace: scores [lists][NK rounded up to 4]
  float2* mz;    // workspace: [rows][C][nsplit] per-split (max, normaliser) of each centroid
  int32_t* count;
  int32_t* kv_idx;
  float* inv_pi;
  float* pi_out;  // may be null
  // per-cluster lists: count / kv_idx / inv_pi above are then the workspace lists
  // [rows * C][cap], and the union goes to ucount / uidx / uw
  int per_cluster;
  uint8_t* label;  // [rows][Bq] last k-means assignment, may be null
  int32_t* ucount;
  int32_t* uidx;
  float* uw;
  int ucap;
};

struct AttendLaunch {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* count;
  const int32_t* kv_idx;
  const float* inv_pi;
  void* o;
  int L, d, Bq, Bk, NQ, NK, rows, cap, out_bf16;
  float scale_log2;  // softmax scale times log2(e)
  // per-cluster lists (null wc: one list per row): kv_idx is the union, wc[row][cap][C]
  // the per-cluster weights, label[row][Bq] each query's cluster (null label with C = 2:
  // the 128-query row is two 64-query blocks and cluster j holds the queries of block j)
  const float* wc;
  const uint8_t* label;
  int C;
  // work queues of the persistent grid (null: one workgroup per row pair): 8 counters,
  // zeroed on the stream before the attention kernel; grid_limit workgroups (the CU count)
  int32_t* queue;
  int grid_limit;
};

// Pairs of 64-query blocks as 128-query rows: row (bh, i) of NQo = ceil(L/128) takes
// the lists of 64-query rows bh*NQi + 2i and, if 2i + 1 < NQi, bh*NQi + 2i + 1, and
// leaves their union (ascending) with one weight per (entry, block), 0 where that
// block's list lacks the entry.
struct PairUnionLaunch {
  const int32_t* count;   // [BH * NQi]
  const int32_t* kv_idx;  // [BH * NQi][cap]
  const float* inv_pi;
  int cap, NK, NQi, NQo, rows_out;
  int32_t* ucount;        // [rows_out]
  int32_t* uidx;          // [rows_out][ucap]
  float* uw;              // [rows_out][ucap][2]
  int ucap;
};

struct QuantFp8Launch {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int BH, L, NK, qk_int8;
  uint8_t* q8;
  float* sq;
  uint8_t* k8;
  float* sk;
  float* kbar;
  uint8_t* v8t;
  float* sv;
  uint16_t* mu;
  double* ksum_part;   // workspace: [BH][ceil(NK/16)][128]
  float* vmax_part;    // workspace: [BH][ceil(NK/16)][128]
  uint16_t* mu_nat;    // workspace: [BH][NK][128] bf16
};

struct AttendFp8Launch {
  const uint8_t* q8;
  const float* sq;
  const uint8_t* k8;
  const float* sk;
  const uint8_t* v8t;
  const float* sv;
  const uint16_t* mu;
  const int32_t* count;
  const int32_t* kv_idx;
  const float* inv_pi;
  void* o;
  int L, NQ, NK, rows, cap, out_bf16, qk_int8;
  float scale_log2;
};

// Number of block-range splits of the logit product (and the 32-block tiles per
// split), chosen so the launch has at least ~2048 workgroups.
inline int logit_splits(int NQ, int C, int BH, int NKp, int* tiles_per_split) {
  const int mtiles = (NQ * C + 127) / 128;
  const int ntile_all = NKp / 32;
  int nsplit = (2048 + mtiles * BH - 1) / (mtiles * BH);
  nsplit = nsplit < 1 ? 1 : (nsplit > ntile_all ? ntile_all : nsplit);
  const int per = (ntile_all + nsplit - 1) / nsplit;
  *tiles_per_split = per;
  return (ntile_all + per - 1) / per;
}

// ev: null, or kSelectEvents events recorded on st before the first kernel and
// after each of the selection's kernels (measurement only)
constexpr int kSelectEvents = 6;
hipError_t launch_select(const SelectLaunch& a, hipStream_t st, hipEvent_t* ev = nullptr);
hipError_t configure_select_kernels();
hipError_t launch_attend(const AttendLaunch& a, hipStream_t st, bool dense);
hipError_t launch_attend_pp(const AttendLaunch& a, hipStream_t st, bool dense);
hipError_t launch_pair_union(const PairUnionLaunch& a, hipStream_t st);
hipError_t launch_quantize_fp8(const QuantFp8Launch& a, hipStream_t st);
hipError_t launch_attend_fp8(const AttendFp8Launch& a, hipStream_t st, bool dense);

}  // namespace absa
