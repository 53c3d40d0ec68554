// C-ABI entry points: argument validation, workspace layout, launches on the
// caller's stream.  Declarations and the contract are in include/absa.h.
#include <cmath>
#include <cstdint>
#include <cstddef>
#include <mutex>

#include "absa.h"
#include "absa_launch.h"

// Fixed selection workspace of absa_select_noalloc, one copy per device
// (module-scope device memory, held until the process ends).  Host code never
// passes `scratch` itself to a kernel: on the host that name is only a stand-in
// for the symbol, and its device address, different on every device, comes from
// hipGetSymbolAddress with that device current (scratch_ptr below).
static constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxNK = 12288;  // the sampler holds a row in the registers of at most 4 waves, the union a word per block in LDS
constexpr size_t kWsAlign = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Dims {
  int64_t BH, rows;
  int NQ, NK, NKp;
};

absa_status check_problem(const absa_problem* p, Dims* dm) {
  if (!p) return ABSA_ERR_INVALID_ARG;
  if (p->B <= 0 || p->H <= 0 || p->L <= 0 || p->d <= 0 || p->T <= 0 || p->Hs <= 0 || p->Ws <= 0 ||
      p->q_block <= 0 || p->kv_block <= 0)
    return ABSA_ERR_SHAPE;
  if ((int64_t)p->T * p->Hs * p->Ws != (int64_t)p->L) return ABSA_ERR_SHAPE;
  if (std::isnan(p->scale) || std::isinf(p->scale)) return ABSA_ERR_INVALID_ARG;
  if (p->out_bf16 != 0 && p->out_bf16 != 1) return ABSA_ERR_INVALID_ARG;
  if (p->d != 64 && p->d != 128) return ABSA_ERR_UNSUPPORTED;
  if (p->q_block != 64 && p->q_block != 128) return ABSA_ERR_UNSUPPORTED;
  if (p->kv_block != 16 && p->kv_block != 32 && p->kv_block != 64 && p->kv_block != 128)
    return ABSA_ERR_UNSUPPORTED;
  const int64_t BH = (int64_t)p->B * p->H;
  // element offsets are computed in 64-bit; row and key indices in 32-bit
  if (BH * (int64_t)p->L * p->d > (int64_t(1) << 46)) return ABSA_ERR_UNSUPPORTED;
  const int NQ = (p->L + p->q_block - 1) / p->q_block;
  const int NK = (p->L + p->kv_block - 1) / p->kv_block;
  if (BH * NQ > INT32_MAX / 2) return ABSA_ERR_UNSUPPORTED;
  if (dm) {
    dm->BH = BH;
    dm->NQ = NQ;
    dm->NK = NK;
    dm->NKp = (NK + 63) / 64 * 64;
    dm->rows = BH * NQ;
  }
  return ABSA_OK;
}

struct SelParams {
  float keep, alpha;
  int C, Tk, mode;
};

absa_status check_params(const absa_problem* p, const absa_select_params* s, SelParams* out) {
  if (!s) return ABSA_ERR_INVALID_ARG;
  if (!(s->keep > 0.f && s->keep <= 1.f)) return ABSA_ERR_INVALID_ARG;  // also rejects NaN
  if (std::isnan(s->select_scale_log2) || std::isinf(s->select_scale_log2)) return ABSA_ERR_INVALID_ARG;
  if (s->mode < ABSA_SEL_SIP || s->mode > ABSA_SEL_ALL) return ABSA_ERR_INVALID_ARG;
  const int C = s->clusters == 0 ? 4 : s->clusters;
  const int Tk = s->kmeans_steps == 0 ? 3 : s->kmeans_steps;
  if (C < 0 || Tk < 0 || Tk > 64) return ABSA_ERR_INVALID_ARG;
  if (C != 1 && C != 2 && C != 4 && C != 8) return ABSA_ERR_UNSUPPORTED;
  if (C > p->q_block) return ABSA_ERR_UNSUPPORTED;
  const float scale = p->scale > 0.f ? p->scale : 1.0f / std::sqrt((float)p->d);
  const float alpha = s->select_scale_log2 > 0.f ? s->select_scale_log2
                                                 : (float)((double)scale * 1.4426950408889634);
  if (out) *out = SelParams{s->keep, alpha, C, Tk, s->mode};
  return ABSA_OK;
}

constexpr int kWsRegions = 7;  // the first 5 are published by absa_select_workspace_layout

struct WsLayout {
  size_t off[kWsRegions];
  size_t total;
};

// Regions: kbar^T, centroids, cluster sizes, scores [lists][NKs] (NKs = NK
// rounded up to 4; one list per row, or per (row, cluster) for per-cluster
// lists), the logit slot (SIZE_MAX: logits are never stored), per-split (max,
// normaliser), the block means' bf16 halves in operand order.
WsLayout ws_layout(const absa_problem* p, const Dims& dm, int C, int lists_per_row) {
  WsLayout w;
  const size_t NKs = (size_t)((dm.NK + 3) & ~3);
  size_t o = 0;
  w.off[0] = o;
  o = align_up(o + (size_t)dm.BH * p->d * dm.NKp * sizeof(float), kWsAlign);
  w.off[1] = o;
  o = align_up(o + (size_t)dm.rows * C * p->d * sizeof(float), kWsAlign);
  w.off[2] = o;
  o = align_up(o + (size_t)dm.rows * C * sizeof(int32_t), kWsAlign);
  w.off[3] = o;
  o = align_up(o + (size_t)dm.rows * lists_per_row * NKs * sizeof(float), kWsAlign);
  w.off[4] = SIZE_MAX;
  w.off[5] = o;
  int per;
  const int nsplit = absa::logit_splits(dm.NQ, C, (int)dm.BH, dm.NKp, &per);
  o = align_up(o + (size_t)dm.rows * C * nsplit * 2 * sizeof(float), kWsAlign);
  w.off[6] = o;
  o = align_up(o + (size_t)2 * dm.BH * dm.NKp * p->d * sizeof(uint16_t), kWsAlign);
  w.total = o;
  return w;
}

// per-cluster selection: the standard regions with scores for every (row, cluster),
// then the clusters' own lists [rows * C][NK] (count, index, weight)
struct WsClusters {
  WsLayout base;
  size_t ccount, cidx, cw, total;
};

WsClusters ws_layout_clusters(const absa_problem* p, const Dims& dm, int C) {
  WsClusters w;
  w.base = ws_layout(p, dm, C, C);
  size_t o = w.base.total;
  w.ccount = o;
  o = align_up(o + (size_t)dm.rows * C * sizeof(int32_t), kWsAlign);
  w.cidx = o;
  o = align_up(o + (size_t)dm.rows * C * dm.NK * sizeof(int32_t), kWsAlign);
  w.cw = o;
  o = align_up(o + (size_t)dm.rows * C * dm.NK * sizeof(float), kWsAlign);
  w.total = o;
  return w;
}

absa_status check_cluster_lists(const absa_cluster_lists* l, int NK, int C) {
  if (!l || !l->count || !l->kv_idx || !l->w || !l->label) return ABSA_ERR_INVALID_ARG;
  if (!aligned(l->count, 4) || !aligned(l->kv_idx, 4) || !aligned(l->w, 4)) return ABSA_ERR_ALIGNMENT;
  if (l->cap < NK) return ABSA_ERR_SHAPE;
  if (l->clusters != C) return ABSA_ERR_SHAPE;
  return ABSA_OK;
}

absa_status check_lists(const absa_blocklist* l, bool need_cap_nk, int NK) {
  if (!l || !l->count || !l->kv_idx || !l->inv_pi) return ABSA_ERR_INVALID_ARG;
  if (!aligned(l->count, 4) || !aligned(l->kv_idx, 4) || !aligned(l->inv_pi, 4)) return ABSA_ERR_ALIGNMENT;
  if (l->cap <= 0) return ABSA_ERR_SHAPE;
  if (need_cap_nk && l->cap < NK) return ABSA_ERR_SHAPE;
  return ABSA_OK;
}

// FP8 path: d = 128, Bk = 16 (and Bq = 128 for the attention step)
absa_status check_fp8_problem(const absa_problem* p, Dims* dm, bool attend) {
  absa_status st = check_problem(p, dm);
  if (st != ABSA_OK) return st;
  if (p->d != 128 || p->kv_block != 16) return ABSA_ERR_UNSUPPORTED;
  if (attend && p->q_block != 128) return ABSA_ERR_UNSUPPORTED;
  // byte offsets inside one head's operands are 32-bit
  if ((int64_t)p->L * 128 > INT32_MAX / 2) return ABSA_ERR_UNSUPPORTED;
  return ABSA_OK;
}

absa_status check_fp8_operands(const absa_fp8_operands* o) {
  if (!o || !o->q8 || !o->sq || !o->k8 || !o->sk || !o->kbar || !o->v8t || !o->sv || !o->mu)
    return ABSA_ERR_INVALID_ARG;
  const void* ps[] = {o->q8, o->sq, o->k8, o->sk, o->kbar, o->v8t, o->sv, o->mu};
  for (const void* p : ps)
    if (!aligned(p, 16)) return ABSA_ERR_ALIGNMENT;
  if (o->qk_int8 != 0 && o->qk_int8 != 1) return ABSA_ERR_INVALID_ARG;
  return ABSA_OK;
}

struct Fp8Ws {
  size_t ksum, vmax, mu_nat, total;
};

Fp8Ws fp8_ws(const Dims& dm) {
  const size_t nchunk = (size_t)(dm.NK + 15) / 16;
  Fp8Ws w;
  size_t o = 0;
  w.ksum = o;
  o = align_up(o + (size_t)dm.BH * nchunk * 128 * sizeof(double), kWsAlign);
  w.vmax = o;
  o = align_up(o + (size_t)dm.BH * nchunk * 128 * sizeof(float), kWsAlign);
  w.mu_nat = o;
  o = align_up(o + (size_t)dm.BH * dm.NK * 128 * sizeof(uint16_t), kWsAlign);
  w.total = o;
  return w;
}

std::once_flag g_attr_once;
hipError_t g_attr_err = hipSuccess;

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, looked up once per device.
hipError_t scratch_ptr(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || !aligned(p, kWsAlign)) return hipErrorInvalidValue;
    g_scratch_ptr[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int32_t absa_version(void) { return ABSA_VERSION; }

const char* absa_status_string(int32_t status) {
  switch (status) {
    case ABSA_OK: return "ok";
    case ABSA_ERR_INVALID_ARG: return "invalid argument";
    case ABSA_ERR_SHAPE: return "inconsistent shape";
    case ABSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case ABSA_ERR_WORKSPACE: return "workspace missing or too small";
    case ABSA_ERR_HIP: return "HIP runtime error";
    case ABSA_ERR_ALIGNMENT: return "misaligned pointer";
    case ABSA_ERR_TOO_LARGE: return "problem needs more than the library's fixed scratch buffer (64 MiB)";
    default: return "unknown status";
  }
}

absa_status absa_num_blocks(const absa_problem* prob, int32_t* nq, int32_t* nk) {
  if (!nq || !nk) return ABSA_ERR_INVALID_ARG;
  Dims dm;
  absa_status st = check_problem(prob, &dm);
  if (st != ABSA_OK) return st;
  *nq = dm.NQ;
  *nk = dm.NK;
  return ABSA_OK;
}

absa_status absa_select_workspace(const absa_problem* prob, const absa_select_params* params,
                                  size_t* bytes) {
  if (!bytes) return ABSA_ERR_INVALID_ARG;
  Dims dm;
  SelParams sp;
  absa_status st = check_problem(prob, &dm);
  if (st != ABSA_OK) return st;
  st = check_params(prob, params, &sp);
  if (st != ABSA_OK) return st;
  *bytes = ws_layout(prob, dm, sp.C, 1).total;
  return ABSA_OK;
}

absa_status absa_select_workspace_layout(const absa_problem* prob, const absa_select_params* params,
                                         size_t* offsets) {
  if (!offsets) return ABSA_ERR_INVALID_ARG;
  Dims dm;
  SelParams sp;
  absa_status st = check_problem(prob, &dm);
  if (st != ABSA_OK) return st;
  st = check_params(prob, params, &sp);
  if (st != ABSA_OK) return st;
  const WsLayout w = ws_layout(prob, dm, sp.C, 1);
  for (int i = 0; i < 5; ++i) offsets[i] = w.off[i];
  return ABSA_OK;
}

static absa::SelectLaunch select_launch(const absa_problem* prob, const absa_select_params* params,
                                        const Dims& dm, const SelParams& sp, const WsLayout& w, char* ws,
                                        const void* q, const void* k) {
  absa::SelectLaunch a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.B = prob->B;
  a.H = prob->H;
  a.L = prob->L;
  a.d = prob->d;
  a.Bq = prob->q_block;
  a.Bk = prob->kv_block;
  a.NQ = dm.NQ;
  a.NK = dm.NK;
  a.NKp = dm.NKp;
  a.C = sp.C;
  a.Tk = sp.Tk;
  a.mode = sp.mode;
  const double nstar = (double)sp.keep * (double)dm.NK;
  a.nstar = (float)nstar;
  const double kst = std::floor(nstar + 0.5);
  a.kstar = (int)(kst < (double)dm.NK ? kst : (double)dm.NK);
  a.alpha = sp.alpha;
  a.key0 = (uint32_t)(params->seed & 0xFFFFFFFFull);
  a.key1 = (uint32_t)(params->seed >> 32);
  a.ctr3 = params->stream;
  a.kbarT = reinterpret_cast<float*>(ws + w.off[0]);
  a.mu = reinterpret_cast<float*>(ws + w.off[1]);
  a.nj = reinterpret_cast<int*>(ws + w.off[2]);
  a.s = reinterpret_cast<float*>(ws + w.off[3]);
  a.mz = reinterpret_cast<float2*>(ws + w.off[5]);
  a.kbh = reinterpret_cast<uint16_t*>(ws + w.off[6]);
  return a;
}

// Validation of absa_select's arguments other than the workspace; fills the
// dimensions, parameters and workspace layout of a valid call.
static absa_status check_select(const absa_problem* prob, const absa_select_params* params, const void* q,
                                const void* k, const absa_blocklist* out, const float* pi_out, Dims* dm,
                                SelParams* sp, WsLayout* w) {
  absa_status st = check_problem(prob, dm);
  if (st != ABSA_OK) return st;
  st = check_params(prob, params, sp);
  if (st != ABSA_OK) return st;
  if (!q || !k) return ABSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16)) return ABSA_ERR_ALIGNMENT;
  if (dm->NK > kMaxNK) return ABSA_ERR_UNSUPPORTED;
  st = check_lists(out, true, dm->NK);
  if (st != ABSA_OK) return st;
  if (pi_out && !aligned(pi_out, 4)) return ABSA_ERR_ALIGNMENT;
  *w = ws_layout(prob, *dm, sp->C, 1);
  return ABSA_OK;
}

// The launches of one selection call into a checked workspace.
static absa_status run_select(const absa_problem* prob, const absa_select_params* params, const Dims& dm,
                              const SelParams& sp, const WsLayout& w, const void* q, const void* k,
                              const absa_blocklist* out, float* pi_out, char* workspace, void* stream) {
  std::call_once(g_attr_once, [] { g_attr_err = absa::configure_select_kernels(); });
  if (g_attr_err != hipSuccess) return ABSA_ERR_HIP;
  absa::SelectLaunch a = select_launch(prob, params, dm, sp, w, workspace, q, k);
  a.count = out->count;
  a.kv_idx = out->kv_idx;
  a.inv_pi = out->inv_pi;
  a.cap = out->cap;
  a.pi_out = pi_out;
  if (!pi_out) a.kbarT = nullptr;  // the fp32 block means are stored only for inspection
  hipError_t e = absa::launch_select(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ABSA_OK : ABSA_ERR_HIP;
}

absa_status absa_select(const absa_problem* prob, const absa_select_params* params, const void* q,
                        const void* k, const absa_blocklist* out, float* pi_out, void* workspace,
                        size_t workspace_bytes, void* stream) {
  Dims dm;
  SelParams sp;
  WsLayout w;
  absa_status st = check_select(prob, params, q, k, out, pi_out, &dm, &sp, &w);
  if (st != ABSA_OK) return st;
  if (!workspace || workspace_bytes < w.total) return ABSA_ERR_WORKSPACE;
  if (!aligned(workspace, kWsAlign)) return ABSA_ERR_ALIGNMENT;
  return run_select(prob, params, dm, sp, w, q, k, out, pi_out, static_cast<char*>(workspace), stream);
}

absa_status absa_select_noalloc(const absa_problem* prob, const absa_select_params* params, const void* q,
                                const void* k, const absa_blocklist* out, float* pi_out, void* stream) {
  Dims dm;
  SelParams sp;
  WsLayout w;
  absa_status st = check_select(prob, params, q, k, out, pi_out, &dm, &sp, &w);
  if (st != ABSA_OK) return st;
  if (w.total > kScratchBytes) return ABSA_ERR_TOO_LARGE;
  char* ws = nullptr;
  if (scratch_ptr(&ws) != hipSuccess) return ABSA_ERR_HIP;
  return run_select(prob, params, dm, sp, w, q, k, out, pi_out, ws, stream);
}

absa_status absa_select_profile(const absa_problem* prob, const absa_select_params* params, const void* q,
                                const void* k, const absa_blocklist* out, void* workspace, size_t workspace_bytes,
                                void* stream, float* kernel_ms, int32_t n_ms) {
  if (!kernel_ms || n_ms < 0) return ABSA_ERR_INVALID_ARG;
  Dims dm;
  SelParams sp;
  WsLayout w;
  absa_status st = check_select(prob, params, q, k, out, nullptr, &dm, &sp, &w);
  if (st != ABSA_OK) return st;
  if (!workspace || workspace_bytes < w.total) return ABSA_ERR_WORKSPACE;
  if (!aligned(workspace, kWsAlign)) return ABSA_ERR_ALIGNMENT;
  std::call_once(g_attr_once, [] { g_attr_err = absa::configure_select_kernels(); });
  if (g_attr_err != hipSuccess) return ABSA_ERR_HIP;
  hipEvent_t ev[absa::kSelectEvents];
  int made = 0;
  hipError_t e = hipSuccess;
  for (; made < absa::kSelectEvents && e == hipSuccess; ++made) e = hipEventCreate(&ev[made]);
  if (e == hipSuccess) {
    absa::SelectLaunch a = select_launch(prob, params, dm, sp, w, static_cast<char*>(workspace), q, k);
    a.count = out->count;
    a.kv_idx = out->kv_idx;
    a.inv_pi = out->inv_pi;
    a.cap = out->cap;
    a.kbarT = nullptr;
    e = absa::launch_select(a, static_cast<hipStream_t>(stream), ev);
  }
  if (e == hipSuccess) e = hipEventSynchronize(ev[absa::kSelectEvents - 1]);
  for (int i = 0; e == hipSuccess && i + 1 < absa::kSelectEvents && i < n_ms; ++i)
    e = hipEventElapsedTime(&kernel_ms[i], ev[i], ev[i + 1]);
  for (int i = 0; i < made; ++i) (void)hipEventDestroy(ev[i]);  // (a failure here changes no result)
  return e == hipSuccess ? ABSA_OK : ABSA_ERR_HIP;
}

absa_status absa_select_clusters_workspace(const absa_problem* prob, const absa_select_params* params,
                                           size_t* bytes) {
  if (!bytes) return ABSA_ERR_INVALID_ARG;
  Dims dm;
  SelParams sp;
  absa_status st = check_problem(prob, &dm);
  if (st != ABSA_OK) return st;
  st = check_params(prob, params, &sp);
  if (st != ABSA_OK) return st;
  *bytes = ws_layout_clusters(prob, dm, sp.C).total;
  return ABSA_OK;
}

absa_status absa_select_clusters(const absa_problem* prob, const absa_select_params* params, const void* q,
                                 const void* k, const absa_cluster_lists* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  Dims dm;
  SelParams sp;
  absa_status st = check_problem(prob, &dm);
  if (st != ABSA_OK) return st;
  st = check_params(prob, params, &sp);
  if (st != ABSA_OK) return st;
  if (!q || !k) return ABSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16)) return ABSA_ERR_ALIGNMENT;
  if (dm.NK > kMaxNK) return ABSA_ERR_UNSUPPORTED;
  st = check_cluster_lists(out, dm.NK, sp.C);
  if (st != ABSA_OK) return st;
  const WsClusters w = ws_layout_clusters(prob, dm, sp.C);
  if (!workspace || workspace_bytes < w.total) return ABSA_ERR_WORKSPACE;
  if (!aligned(workspace, kWsAlign)) return ABSA_ERR_ALIGNMENT;

  std::call_once(g_attr_once, [] { g_attr_err = absa::configure_select_kernels(); });
  if (g_attr_err != hipSuccess) return ABSA_ERR_HIP;

  char* ws = static_cast<char*>(workspace);
  absa::SelectLaunch a = select_launch(prob, params, dm, sp, w.base, ws, q, k);
  a.per_cluster = 1;
  a.kbarT = nullptr;
  a.count = reinterpret_cast<int32_t*>(ws + w.ccount);
  a.kv_idx = reinterpret_cast<int32_t*>(ws + w.cidx);
  a.inv_pi = reinterpret_cast<float*>(ws + w.cw);
  a.cap = dm.NK;
  a.pi_out = nullptr;
  a.label = out->label;
  a.ucount = out->count;
  a.uidx = out->kv_idx;
  a.uw = out->w;
  a.ucap = out->cap;
  hipError_t e = absa::launch_select(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ABSA_OK : ABSA_ERR_HIP;
}

// The bf16 attention kernels address one head's K and V through 32-bit buffer
// offsets, with 0x7FFFFFF0 as the out-of-range base of entries outside a list:
// a head's L*d*2 bytes plus one 64-key tile must stay below it.
static bool head_fits_buffer(const absa_problem* p) {
  return (int64_t)p->L * p->d * 2 <= (int64_t)0x7FFFFFF0 - (int64_t)64 * p->d * 2;
}

// Work queues of the persistent attention grid: 8 counters in a 256-byte region.
constexpr size_t kQueueBytes = 256;

// Workgroups of the persistent grid: one per compute unit of the current device.
static int persistent_grid() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

static absa_status attend_common(const absa_problem* prob, const void* q, const void* k, const void* v,
                                 const absa_blocklist* lists, void* o, void* stream, bool dense,
                                 int32_t* queue = nullptr) {
  Dims dm;
  absa_status st = check_problem(prob, &dm);
  if (st != ABSA_OK) return st;
  if (!head_fits_buffer(prob)) return ABSA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !o) return ABSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return ABSA_ERR_ALIGNMENT;
  if (!dense) {
    st = check_lists(lists, false, dm.NK);
    if (st != ABSA_OK) return st;
  }
  absa::AttendLaunch a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = o;
  a.L = prob->L;
  a.d = prob->d;
  a.Bq = prob->q_block;
  a.Bk = dense ? 64 : prob->kv_block;
  a.NQ = dm.NQ;
  a.NK = dense ? (prob->L + 63) / 64 : dm.NK;
  a.rows = (int)dm.rows;
  a.out_bf16 = prob->out_bf16;
  const float scale = prob->scale > 0.f ? prob->scale : 1.0f / std::sqrt((float)prob->d);
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  if (!dense) {
    a.count = lists->count;
    a.kv_idx = lists->kv_idx;
    a.inv_pi = lists->inv_pi;
    a.cap = lists->cap;
  }
  if (queue && prob->q_block == 128) {
    a.grid_limit = persistent_grid();
    if (a.grid_limit <= 0) return ABSA_ERR_HIP;
    a.queue = queue;
  }
  hipError_t e = absa::launch_attend(a, static_cast<hipStream_t>(stream), dense);
  return e == hipSuccess ? ABSA_OK : ABSA_ERR_HIP;
}

absa_status absa_attend(const absa_problem* prob, const void* q, const void* k, const void* v,
                        const absa_blocklist* lists, void* o, void* stream) {
  return attend_common(prob, q, k, v, lists, o, stream, false);
}

absa_status absa_dense(const absa_problem* prob, const void* q, const void* k, const void* v, void* o,
                       void* stream) {
  return attend_common(prob, q, k, v, nullptr, o, stream, true);
}

absa_status absa_attend_balanced_workspace(size_t* bytes) {
  if (!bytes) return ABSA_ERR_INVALID_ARG;
  *bytes = kQueueBytes;
  return ABSA_OK;
}

absa_status absa_attend_balanced(const absa_problem* prob, const void* q, const void* k, const void* v,
                                 const absa_blocklist* lists, void* o, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  Dims dm;
  absa_status st = check_problem(prob, &dm);
  if (st != ABSA_OK) return st;
  if (!workspace || workspace_bytes < kQueueBytes) return ABSA_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return ABSA_ERR_ALIGNMENT;
  return attend_common(prob, q, k, v, lists, o, stream, false, static_cast<int32_t*>(workspace));
}

absa_status absa_attend_clusters(const absa_problem* prob, const void* q, const void* k, const void* v,
                                 const absa_cluster_lists* lists, void* o, void* stream) {
  Dims dm;
  absa_status st = check_problem(prob, &dm);
  if (st != ABSA_OK) return st;
  if (!head_fits_buffer(prob)) return ABSA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !o) return ABSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return ABSA_ERR_ALIGNMENT;
  if (prob->q_block != 128) return ABSA_ERR_UNSUPPORTED;
  if (!lists) return ABSA_ERR_INVALID_ARG;
  if (lists->clusters != 1 && lists->clusters != 2 && lists->clusters != 4 && lists->clusters != 8)
    return ABSA_ERR_UNSUPPORTED;
  st = check_cluster_lists(lists, dm.NK, lists->clusters);
  if (st != ABSA_OK) return st;
  absa::AttendLaunch a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = o;
  a.L = prob->L;
  a.d = prob->d;
  a.Bq = prob->q_block;
  a.Bk = prob->kv_block;
  a.NQ = dm.NQ;
  a.NK = dm.NK;
  a.rows = (int)dm.rows;
  a.out_bf16 = prob->out_bf16;
  const float scale = prob->scale > 0.f ? prob->scale : 1.0f / std::sqrt((float)prob->d);
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.count = lists->count;
  a.kv_idx = lists->kv_idx;
  a.inv_pi = nullptr;
  a.cap = lists->cap;
  a.wc = lists->w;
  a.label = lists->label;
  a.C = lists->clusters;
  hipError_t e = absa::launch_attend(a, static_cast<hipStream_t>(stream), false);
  return e == hipSuccess ? ABSA_OK : ABSA_ERR_HIP;
}

// Pairs of 64-query blocks: the union lists [rows128] count, [rows128][NK] indices
// and [rows128][NK][2] weights, 256-byte aligned regions.
struct PairWs {
  size_t ucount, uidx, uw, queue, total;
};
static PairWs pair_ws(const absa_problem* p, const Dims& dm) {
  const int64_t NQo = (p->L + 127) / 128;
  const int64_t rows = dm.BH * NQo;
  PairWs w;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  w.ucount = take((size_t)rows * 4);
  w.uidx = take((size_t)rows * dm.NK * 4);
  w.uw = take((size_t)rows * dm.NK * 2 * 4);
  w.queue = take(kQueueBytes);
  w.total = off;
  return w;
}

static absa_status check_pairs_problem(const absa_problem* prob, Dims* dm) {
  absa_status st = check_problem(prob, dm);
  if (st != ABSA_OK) return st;
  if (prob->q_block != 64) return ABSA_ERR_UNSUPPORTED;
  if (!head_fits_buffer(prob)) return ABSA_ERR_UNSUPPORTED;
  if (dm->NK > kMaxNK) return ABSA_ERR_UNSUPPORTED;  // the union keeps a word per block in LDS
  return ABSA_OK;
}

absa_status absa_attend_pairs_workspace(const absa_problem* prob, size_t* bytes) {
  if (!bytes) return ABSA_ERR_INVALID_ARG;
  Dims dm;
  absa_status st = check_pairs_problem(prob, &dm);
  if (st != ABSA_OK) return st;
  *bytes = pair_ws(prob, dm).total;
  return ABSA_OK;
}

absa_status absa_attend_pairs(const absa_problem* prob, const void* q, const void* k, const void* v,
                              const absa_blocklist* lists, void* o, void* workspace, size_t workspace_bytes,
                              void* stream) {
  Dims dm;
  absa_status st = check_pairs_problem(prob, &dm);
  if (st != ABSA_OK) return st;
  if (!q || !k || !v || !o) return ABSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return ABSA_ERR_ALIGNMENT;
  st = check_lists(lists, false, dm.NK);
  if (st != ABSA_OK) return st;
  const PairWs w = pair_ws(prob, dm);
  if (!workspace || workspace_bytes < w.total) return ABSA_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return ABSA_ERR_ALIGNMENT;
  char* ws = static_cast<char*>(workspace);
  const int NQo = (prob->L + 127) / 128;
  absa::PairUnionLaunch u{};
  u.count = lists->count;
  u.kv_idx = lists->kv_idx;
  u.inv_pi = lists->inv_pi;
  u.cap = lists->cap;
  u.NK = dm.NK;
  u.NQi = dm.NQ;
  u.NQo = NQo;
  u.rows_out = (int)(dm.BH * NQo);
  u.ucount = reinterpret_cast<int32_t*>(ws + w.ucount);
  u.uidx = reinterpret_cast<int32_t*>(ws + w.uidx);
  u.uw = reinterpret_cast<float*>(ws + w.uw);
  u.ucap = dm.NK;
  hipError_t e = absa::launch_pair_union(u, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return ABSA_ERR_HIP;
  // the pairs as the rows of a 128-query problem, each query over its own block's list
  absa::AttendLaunch a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = o;
  a.L = prob->L;
  a.d = prob->d;
  a.Bq = 128;
  a.Bk = prob->kv_block;
  a.NQ = NQo;
  a.NK = dm.NK;
  a.rows = u.rows_out;
  a.out_bf16 = prob->out_bf16;
  const float scale = prob->scale > 0.f ? prob->scale : 1.0f / std::sqrt((float)prob->d);
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.count = u.ucount;
  a.kv_idx = u.uidx;
  a.inv_pi = nullptr;
  a.cap = u.ucap;
  a.wc = u.uw;
  a.label = nullptr;
  a.C = 2;
  a.grid_limit = persistent_grid();
  if (a.grid_limit <= 0) return ABSA_ERR_HIP;
  a.queue = reinterpret_cast<int32_t*>(ws + w.queue);
  e = absa::launch_attend(a, static_cast<hipStream_t>(stream), false);
  return e == hipSuccess ? ABSA_OK : ABSA_ERR_HIP;
}

absa_status absa_fp8_workspace(const absa_problem* prob, size_t* bytes) {
  if (!bytes) return ABSA_ERR_INVALID_ARG;
  Dims dm;
  absa_status st = check_fp8_problem(prob, &dm, false);
  if (st != ABSA_OK) return st;
  *bytes = fp8_ws(dm).total;
  return ABSA_OK;
}

absa_status absa_quantize_fp8(const absa_problem* prob, const void* q, const void* k, const void* v,
                              const absa_fp8_operands* out, void* workspace, size_t workspace_bytes,
                              void* stream) {
  Dims dm;
  absa_status st = check_fp8_problem(prob, &dm, false);
  if (st != ABSA_OK) return st;
  if (!q || !k || !v) return ABSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16)) return ABSA_ERR_ALIGNMENT;
  st = check_fp8_operands(out);
  if (st != ABSA_OK) return st;
  const Fp8Ws w = fp8_ws(dm);
  if (!workspace || workspace_bytes < w.total) return ABSA_ERR_WORKSPACE;
  if (!aligned(workspace, kWsAlign)) return ABSA_ERR_ALIGNMENT;
  char* ws = static_cast<char*>(workspace);
  absa::QuantFp8Launch a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.BH = (int)dm.BH;
  a.L = prob->L;
  a.NK = dm.NK;
  a.qk_int8 = out->qk_int8;
  a.q8 = out->q8;
  a.sq = out->sq;
  a.k8 = out->k8;
  a.sk = out->sk;
  a.kbar = out->kbar;
  a.v8t = out->v8t;
  a.sv = out->sv;
  a.mu = out->mu;
  a.ksum_part = reinterpret_cast<double*>(ws + w.ksum);
  a.vmax_part = reinterpret_cast<float*>(ws + w.vmax);
  a.mu_nat = reinterpret_cast<uint16_t*>(ws + w.mu_nat);
  hipError_t e = absa::launch_quantize_fp8(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ABSA_OK : ABSA_ERR_HIP;
}

absa_status absa_attend_fp8(const absa_problem* prob, const absa_fp8_operands* ops,
                            const absa_blocklist* lists, void* o, void* stream) {
  Dims dm;
  absa_status st = check_fp8_problem(prob, &dm, true);
  if (st != ABSA_OK) return st;
  st = check_fp8_operands(ops);
  if (st != ABSA_OK) return st;
  if (!o) return ABSA_ERR_INVALID_ARG;
  if (!aligned(o, 16)) return ABSA_ERR_ALIGNMENT;
  const bool dense = lists == nullptr;
  if (!dense) {
    st = check_lists(lists, false, dm.NK);
    if (st != ABSA_OK) return st;
  }
  absa::AttendFp8Launch a{};
  a.q8 = ops->q8;
  a.sq = ops->sq;
  a.k8 = ops->k8;
  a.sk = ops->sk;
  a.v8t = ops->v8t;
  a.sv = ops->sv;
  a.mu = ops->mu;
  a.o = o;
  a.L = prob->L;
  a.NQ = dm.NQ;
  a.NK = dm.NK;
  a.rows = (int)dm.rows;
  a.out_bf16 = prob->out_bf16;
  a.qk_int8 = ops->qk_int8;
  const float scale = prob->scale > 0.f ? prob->scale : 1.0f / std::sqrt((float)prob->d);
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  if (!dense) {
    a.count = lists->count;
    a.kv_idx = lists->kv_idx;
    a.inv_pi = lists->inv_pi;
    a.cap = lists->cap;
  }
  hipError_t e = absa::launch_attend_fp8(a, static_cast<hipStream_t>(stream), dense);
  return e == hipSuccess ? ABSA_OK : ABSA_ERR_HIP;
}

}  // extern "C"
