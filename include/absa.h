/*
 * absa.h -- C ABI of the AB-Attention block-sparse attention library (gfx950).
 *
 * The method (AB-Attention page, edumints blog, section "AB-Attention ve Üç
 * Temel Yeniliği") approximates dense attention softmax(Q K^T / sqrt(d)) V
 * (Cross-Attention glossary page, formula in its opening section) for video
 * diffusion transformers, whose clip is one flattened spatiotemporal token
 * sequence (VC-Attention page, opening section), in three parts:
 *   IBCS  clusters the queries inside each query block, without permuting
 *         tokens, and scores KV blocks from the cluster centroids;
 *   SIP   samples KV blocks with probabilities tied to those scores and
 *         reweights kept blocks by 1/pi in the softmax numerator and
 *         denominator, so a single pass estimates dense attention;
 *   a kernel that packs KV blocks much smaller than a tile into full
 *         matrix-core tiles.
 *
 * The pages fix no formula for IBCS or SIP.  The rules implemented here:
 *   KV block summary   mean of the block's valid keys;
 *   IBCS               Lloyd k-means of the block's query vectors (squared
 *                      Euclidean), C clusters initialised at members
 *                      floor(j*n/C), Tk steps, ties to the lowest cluster,
 *                      empty clusters keep their centroid;
 *   score s_b          sum_j (n_j/n) * nk_b * 2^(l_jb - m_j) / Z_j with
 *                      l_jb = alpha * mu_j . kbar_b, m_j = max_b l_jb, terms
 *                      with l_jb - m_j < -64 dropped, Z_j normalising; the dot
 *                      products split each fp32 operand into a bf16 head and
 *                      tail (hi.hi' + hi.lo' + lo.hi', fp32 sums): exact when
 *                      bf16 holds mu and kbar, ~2^-15 relative otherwise;
 *   inclusion pi_b     min(1, lambda s_b) with sum_b pi_b = keep * NK,
 *                      solved by iterative capping, rounded to fp32;
 *   draw               Philox4x32-10 (Salmon et al., SC'11) with counter
 *                      (b/4, i, b*H+h, stream) and key (seed lo, seed hi),
 *                      word b%4, u = (x >> 8) * 2^-24, keep iff u < pi_b;
 *   weight             w_b = fp32(1 / pi_b);
 *   estimate           o_t = sum_{b in S} w_b sum_{k in b} e^{a_tk} v_k /
 *                            sum_{b in S} w_b sum_{k in b} e^{a_tk},
 *                      a_tk = scale * q_t . k_k (0 for an empty list).
 *
 * Conventions for every entry point:
 *   - Every tensor pointer is a device pointer on the current HIP device.
 *     Struct pointers marked [host] point to host memory.
 *   - Q, K, V are [B, H, L, d] bf16, contiguous, unpadded, 16-byte aligned.
 *     Blocks are contiguous token ranges in the caller's order: query block i
 *     holds tokens [i*Bq, min(L, (i+1)*Bq)), KV block b holds
 *     [b*Bk, min(L, (b+1)*Bk)).  The last blocks may be partial; tails are
 *     masked inside the kernels.
 *   - A "row" is one (b, h, query block) triple; rows are ordered
 *     (b*H + h)*NQ + i.
 *   - The caller allocates and owns every buffer; the library allocates no
 *     device memory and keeps no mutable global state (the one exception is
 *     the fixed module-scope buffer of absa_select_noalloc, below).
 *   - Calls only enqueue work on `stream` (a hipStream_t; NULL is the null
 *     stream) and never synchronise.  Results are valid once the caller
 *     synchronises with that stream.
 *   - Arguments are validated before any launch; a call that fails validation
 *     returns an error code and has no side effects.  A failed launch returns
 *     ABSA_ERR_HIP.  No C++ exception crosses this interface.
 */
#ifndef ABSA_H_
#define ABSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ABSA_VERSION 10000 /* major*10000 + minor*100 + patch */

typedef enum absa_status {
  ABSA_OK = 0,
  ABSA_ERR_INVALID_ARG = -1, /* null pointer, NaN or out-of-range scalar       */
  ABSA_ERR_SHAPE = -2,       /* inconsistent sizes (e.g. T*Hs*Ws != L)          */
  ABSA_ERR_UNSUPPORTED = -3, /* valid but not implemented (d, block sizes, C)   */
  ABSA_ERR_WORKSPACE = -4,   /* workspace missing or too small                  */
  ABSA_ERR_HIP = -5,         /* a HIP runtime call or a launch failed           */
  ABSA_ERR_ALIGNMENT = -6,   /* a pointer is not aligned as required            */
  ABSA_ERR_TOO_LARGE = -7    /* needs more than absa_select_noalloc's fixed
                                64 MiB scratch buffer                           */
} absa_status;

typedef enum absa_sel_mode {
  ABSA_SEL_SIP = 0,  /* Poisson sampling with 1/pi weights (the method)       */
  ABSA_SEL_TOPK = 1, /* k* = min(NK, floor(keep*NK + 1/2)) highest scores,
                        ties to the lower block index, weight 1 (truncation
                        baseline named in the page's "Dikkat Darboğazı"
                        section)                                             */
  ABSA_SEL_ALL = 2   /* every block, weight 1 (equals dense attention)        */
} absa_sel_mode;

typedef struct absa_problem {
  int32_t B, H, L, d;        /* d in {64, 128}                                 */
  int32_t T, Hs, Ws;         /* token grid; T*Hs*Ws must equal L               */
  int32_t q_block;           /* Bq in {64, 128}                                */
  int32_t kv_block;          /* Bk in {16, 32, 64, 128}                        */
  float scale;               /* softmax scale sigma; <= 0 selects 1/sqrt(d)    */
  int32_t out_bf16;          /* 0: O is fp32, 1: O is bf16                      */
} absa_problem;

typedef struct absa_select_params {
  float keep;                /* expected kept fraction of KV blocks, (0, 1]    */
  int32_t clusters;          /* C in {1, 2, 4, 8}, C <= Bq; 0 selects 4         */
  int32_t kmeans_steps;      /* Tk in [1, 64]; 0 selects 3                      */
  float select_scale_log2;   /* alpha; <= 0 selects scale * log2(e)            */
  uint64_t seed;             /* Philox key                                     */
  uint32_t stream;           /* Philox counter word 3 (e.g. layer or step id)  */
  int32_t mode;              /* absa_sel_mode                                  */
} absa_select_params;

/* Per-row block lists.  count[rows]; kv_idx and inv_pi are [rows][cap], row r
 * holding count[r] entries with ascending unique block indices < NK and
 * weights >= 1.  absa_select writes them (cap must be >= NK); absa_attend
 * accepts any lists in this format (entries with an index >= NK are skipped,
 * counts are clamped to [0, cap]).  All three pointers 4-byte aligned. */
typedef struct absa_blocklist {
  int32_t* count;
  int32_t* kv_idx;
  float* inv_pi;
  int32_t cap;
} absa_blocklist;

/* Library version (ABSA_VERSION of the build). */
int32_t absa_version(void);

/* Static text for a status code; never NULL. */
const char* absa_status_string(int32_t status);

/* NQ = ceil(L/Bq) and NK = ceil(L/Bk) for a valid problem ([host] pointers).
 * Passage: AB-Attention page, section "AB-Attention ve Üç Temel Yeniliği", IBCS item (query
 * blocks are formed without permuting tokens, so blocks are contiguous token
 * ranges of the clip's own order). */
absa_status absa_num_blocks(const absa_problem* prob, int32_t* nq, int32_t* nk);

/* Bytes of device workspace absa_select needs ([host] pointers): the IBCS
 * intermediates (block means, centroids, scores) of AB-Attention page, section "AB-Attention ve Üç Temel Yeniliği",
 * IBCS item. */
absa_status absa_select_workspace(const absa_problem* prob, const absa_select_params* params,
                                  size_t* bytes);

/* Byte offsets inside the workspace of absa_select's intermediates, left
 * there for inspection by a successful absa_select call:
 *   offsets[0]  kbar^T  fp32 [B*H][d][NKp]  block mean keys, NKp = NK rounded up to 64
 *   offsets[1]  mu      fp32 [rows][C][d]   final centroids
 *   offsets[2]  n_j     int32 [rows][C]     final cluster sizes
 *   offsets[3]  s       fp32 [rows][NKs]    block scores, NKs = NK rounded up to 4 (zeros past NK)
 *   offsets[4]  SIZE_MAX: the block logits alpha * mu_j . kbar_b are formed on
 *               chip and never stored
 * mu, n_j and s are written by every call; kbar^T only by calls with a
 * non-NULL pi_out (the inspection mode), since the lists do not need it.
 * ([host] pointers; offsets has 5 entries).  Passage: as absa_select. */
absa_status absa_select_workspace_layout(const absa_problem* prob, const absa_select_params* params,
                                         size_t* offsets);

/* Block selection (IBCS + SIP, or TOPK / ALL): reads Q and K, writes the
 * lists in `out` ([host] struct, device arrays) and, when pi_out is not NULL,
 * the fp32 inclusion probability of every block, [rows][NK] (SIP: pi_b;
 * TOPK: 1 for kept, 0 otherwise; ALL: 1).  Requires NK <= 12288.
 * workspace: device memory of at least absa_select_workspace() bytes, 256-byte
 * aligned, owned by the caller, contents on entry ignored.
 * Passages: AB-Attention page, section "AB-Attention ve Üç Temel Yeniliği",
 * IBCS item (scores from clusters of each query block) and SIP item (blocks
 * sampled in proportion to those scores, weight 1/pi); TOPK is the truncation
 * of the same page's section "Video Difüzyon Modellerinde Dikkat (Attention)
 * Darboğazı" (pruned blocks leave the softmax), ALL its dense attention. */
absa_status absa_select(const absa_problem* prob, const absa_select_params* params, const void* q,
                        const void* k, const absa_blocklist* out, float* pi_out, void* workspace,
                        size_t workspace_bytes, void* stream);

/* absa_select without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, serving loops, harnesses
 * that forbid allocation).  The selection workspace is a fixed 64 MiB buffer in
 * the library's module-scope device memory, one per device, set up on the
 * first call on that device and held until the process ends; this call itself
 * allocates nothing.  Problems whose workspace (absa_select_workspace) exceeds
 * 64 MiB return ABSA_ERR_TOO_LARGE before any launch.  Outputs, arguments and
 * errors are those of absa_select; the buffer's intermediates are not
 * published.  Every call on one device shares that device's buffer: calls
 * whose work overlaps on one device (on different streams, or from several
 * threads without ordering) race and give undefined lists; calls on one
 * stream are ordered and safe.  A failed lookup of the buffer returns
 * ABSA_ERR_HIP. */
absa_status absa_select_noalloc(const absa_problem* prob, const absa_select_params* params, const void* q,
                                const void* k, const absa_blocklist* out, float* pi_out, void* stream);

/* Measurement: absa_select (without probabilities) with a HIP event recorded
 * on `stream` before and after each of its five kernels -- block means, k-means,
 * logit normalisers, scores, sampling -- and the time of each, in ms and in that
 * order, written to the first min(n_ms, 5) entries of kernel_ms ([host]).  The
 * call waits for the selection to finish; the lists are those absa_select
 * gives.  Arguments and errors as absa_select; n_ms < 0 or a NULL kernel_ms
 * is ABSA_ERR_INVALID_ARG, a failed event call ABSA_ERR_HIP.  Passage: as
 * absa_select. */
absa_status absa_select_profile(const absa_problem* prob, const absa_select_params* params, const void* q,
                                const void* k, const absa_blocklist* out, void* workspace, size_t workspace_bytes,
                                void* stream, float* kernel_ms, int32_t n_ms);

/* Block-sparse attention over given lists (the estimate above): for every
 * valid query of row r, attends to the keys of the blocks listed for r with
 * their weights.  o is [B, H, L, d] (fp32, or bf16 if out_bf16), 16-byte
 * aligned; only valid query rows are written.  `lists` is a [host] struct.
 * Passages: AB-Attention page, section "AB-Attention ve Üç Temel Yeniliği",
 * SIP item (the 1/pi weights enter the softmax numerator and denominator, one
 * pass estimates dense attention) and kernel item (KV blocks much smaller than
 * a tile are packed into full matrix-core tiles); the attention formula of the
 * Cross-Attention glossary page's opening section. */
absa_status absa_attend(const absa_problem* prob, const void* q, const void* k, const void* v,
                        const absa_blocklist* lists, void* o, void* stream);

/* Bytes of device workspace absa_attend_balanced needs (its work queues),
 * written to *bytes ([host]); NULL bytes is ABSA_ERR_INVALID_ARG. */
absa_status absa_attend_balanced_workspace(size_t* bytes);

/* absa_attend on a persistent grid, for 128-query blocks: one workgroup per
 * compute unit takes row pairs from eight work queues, one per XCD, holding
 * the pairs absa_attend's one-workgroup-per-pair grid deals to that XCD, in
 * the same order; once its own queue is empty it takes from the others.  The
 * output is bit-identical to absa_attend's; the XCDs, which do not all run at
 * the same clock, then finish together instead of the faster ones idling at
 * the end.  For 64-query blocks it runs as absa_attend (workspace unused).
 * workspace: at least absa_attend_balanced_workspace() bytes of device
 * memory, 256-byte aligned, contents on entry ignored (the call clears its
 * queues on `stream` before the attention kernel); calls that share a
 * workspace must not overlap.  Errors as absa_attend, plus ABSA_ERR_WORKSPACE
 * (NULL or too small) and ABSA_ERR_ALIGNMENT.  Passages: as absa_attend. */
absa_status absa_attend_balanced(const absa_problem* prob, const void* q, const void* k, const void* v,
                                 const absa_blocklist* lists, void* o, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* Bytes of device workspace absa_attend_pairs needs ([host] pointers): the union
 * lists of each pair of 64-query blocks, ceil(L/128) per head, NK entries each
 * (count, indices and two weights per entry), and the work queues of its
 * persistent grid (as absa_attend_balanced).  Same problem rules as
 * absa_attend_pairs. */
absa_status absa_attend_pairs_workspace(const absa_problem* prob, size_t* bytes);

/* absa_attend for 64-query blocks (Bq = 64, else ABSA_ERR_UNSUPPORTED; NK <=
 * 12288), on the 128-query two-row kernel: query blocks 2i and 2i + 1 of a
 * head form one 128-query row (tokens [128 i, 128 i + 128)) that walks the
 * ascending union of their two lists, each entry carrying both blocks'
 * weights, 0 for a block whose list lacks it; each query takes the weight of
 * its own block, so it attends over exactly its block's list with its
 * weights, as in absa_attend (the same result up to the order of fp32 sums).
 * Lists in absa_attend's format (ascending unique indices; entries >= NK
 * skipped).  workspace: at least absa_attend_pairs_workspace() bytes,
 * 256-byte aligned, contents on entry ignored, overwritten.  Passages: as
 * absa_attend; the union with per-member weights is the per-cluster hand-over
 * below (PIVOT page, section "PIVOT'un arkasındaki iki gözlem"), here with the
 * two query blocks as the groups. */
absa_status absa_attend_pairs(const absa_problem* prob, const void* q, const void* k, const void* v,
                              const absa_blocklist* lists, void* o, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Dense attention softmax(scale Q K^T) V over all L keys, same layouts.
 * Passages: the 3D full attention of the AB-Attention page's section "Video
 * Difüzyon Modellerinde Dikkat (Attention) Darboğazı" (the quantity the
 * estimate approximates), written as in the Cross-Attention glossary page's
 * opening section. */
absa_status absa_dense(const absa_problem* prob, const void* q, const void* k, const void* v, void* o,
                       void* stream);

/* ---------------------------------------------------------------------------
 * Per-cluster block lists.  The PIVOT page (section "PIVOT'un arkasındaki iki
 * gözlem") scores one proxy per group of queries and then refines the proxy's
 * candidate list for each member of the group; here the groups are the IBCS
 * clusters of each query block and the refinement is one SIP sample per
 * cluster:
 *   score      s_b^(j) = nk_b 2^(l_jb - m_j) / Z_j (cluster j's own block
 *              distribution; the shared score is the mixture over j);
 *   sample     per cluster: capped pi^(j) with sum = keep * NK, Philox counter
 *              (b/4, i*C + j, b*H+h, stream), weight fp32(1/pi); a cluster with
 *              no member gets an empty list (TOPK and ALL modes likewise per
 *              cluster);
 *   estimate   each query over its own cluster's list and weights.
 * With C = 1 the sample equals the shared one.  Attention walks the union of a
 * row's lists once, in the 128-query two-row kernel (Bq = 128). */
typedef struct absa_cluster_lists {
  int32_t* count;   /* [rows]             entries in the row's union list                */
  int32_t* kv_idx;  /* [rows][cap]        ascending union of the clusters' samples       */
  float* w;         /* [rows][cap][C]     weight of entry e for cluster j, 0 if cluster j
                                          did not draw the block                         */
  uint8_t* label;   /* [rows][Bq]         cluster of each query of the row (the last
                                          k-means assignment; 0 past the block's queries) */
  int32_t cap;      /* >= NK                                                             */
  int32_t clusters; /* C; must equal the selection's cluster count                       */
} absa_cluster_lists;

/* Bytes of device workspace absa_select_clusters needs ([host] pointers).
 * Passage: the PIVOT page, section "PIVOT'un arkasındaki iki gözlem". */
absa_status absa_select_clusters_workspace(const absa_problem* prob, const absa_select_params* params,
                                           size_t* bytes);

/* Per-cluster selection into `out` ([host] struct, device arrays, 4-byte
 * aligned).  Same requirements and workspace rules as absa_select (NK <=
 * 12288); the workspace is larger (scores and lists of every cluster).
 * Passages: the PIVOT page, section "PIVOT'un arkasındaki iki gözlem" (one
 * proxy per query group, its candidates refined per member), with the IBCS
 * clusters and SIP draws of AB-Attention page, section "AB-Attention ve Üç Temel Yeniliği". */
absa_status absa_select_clusters(const absa_problem* prob, const absa_select_params* params, const void* q,
                                 const void* k, const absa_cluster_lists* out, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Attention over per-cluster lists: query t of row r over the blocks its
 * cluster drew, with that cluster's weights.  Layouts as for absa_attend;
 * requires Bq = 128.  Passages: as absa_select_clusters and absa_attend. */
absa_status absa_attend_clusters(const absa_problem* prob, const void* q, const void* k, const void* v,
                                 const absa_cluster_lists* lists, void* o, void* stream);

/* ---------------------------------------------------------------------------
 * FP8 (E4M3) variant of the attention step.  The VC-Attention page (section
 * "İki darboğaz") puts most low-bit attention error in the value term, removes
 * part of it by subtracting a per-block mean of V before quantising, and writes
 * the softmax probabilities as E4M3 bytes directly, with one fused multiply-add
 * per element, because an E4M3 byte is close to a scaled log2 of its value
 * ("ExpCast"); section "Ölçümler" says such a kernel composes with sparse
 * attention.  The rules implemented here (E4M3 = OCP E4M3FN: bias 7, largest
 * finite 448; every scale s = 2^e with e the smallest integer for which
 * max|x| <= 448 s, 1 for all-zero sets):
 *   Q      per token: s_Q[t] from max_c |q[t][c]|, code = e4m3_rne(q / s_Q);
 *   K      kbar[c] = fp32(sum_t k[t][c] / L) (mean over the head's L tokens;
 *          it cancels in every query's softmax); per KV block b:
 *          s_K[b] from max |k - kbar| over its valid keys, code =
 *          e4m3_rne((k - kbar) / s_K) with k - kbar rounded to fp32;
 *   V      mu_hat[b][c] = bf16(fp32(mean of block b's valid keys)); residual
 *          r = v - mu_hat (fp32); per channel c of the head: s_V[c] from
 *          max_t |r[t][c]|, code = e4m3_rne(r / s_V);
 *   P      y = 8 (l - m) + 120 in fp32 (one fused multiply-add from the dot
 *          product of the codes) with l = scale log2(e) s_Q s_K (q8.k8)
 *          + log2 w_b and m, per query, the smallest integer that keeps
 *          every y of the row's kept keys at or below 120 (so m = ceil(max l)
 *          up to the roundings of y, independent of the list's order);
 *          p = e4m3 value of the byte sat_u8(rne(y)).  The kernel reaches m
 *          through a running reference that rises by whole octaves, so a term
 *          formed under an earlier, lower reference can differ from its value
 *          under m only below E4M3's normal range (bytes < 8, more than 14
 *          octaves under the row's largest term);
 *   O      o_t = sum_k p_k (mu_hat + s_V dec(code_k)) / sum_k p_k (0 for an
 *          empty list).
 *   QK     optionally INT8 instead of E4M3 (the page builds on earlier 8-bit
 *          kernels that smooth K and quantise QK to integers): the same Q and
 *          K scaling with 127 in place of 448, codes clip(rne(x / s), -127, 127),
 *          exact integer dot products.
 * Supported shape: d = 128, Bq = 128, Bk = 16.
 */

/* Quantised operands of one problem; every pointer is a device pointer owned
 * by the caller, 16-byte aligned.  NK = ceil(L/16). */
typedef struct absa_fp8_operands {
  uint8_t* q8;    /* [B,H,L,128]      E4M3 codes of Q                              */
  float* sq;      /* [B,H,L]          s_Q per token                                */
  uint8_t* k8;    /* [B,H,L,128]      E4M3 codes of k - kbar                       */
  float* sk;      /* [B,H,NK]         s_K per KV block                             */
  float* kbar;    /* [B,H,128]        per-head key mean                            */
  uint8_t* v8t;   /* [B,H,NK,128,16]  E4M3 codes of v - mu_hat, block by block with
                                      the 16 keys of a channel contiguous (keys
                                      past L hold code 0)                          */
  float* sv;      /* [B,H,128]        s_V per channel                              */
  uint16_t* mu;   /* [B,H,NK,32,4]    bf16 mu_hat[b][32 j + i] / s_V[32 j + i] at
                                      [b][i][j], i.e. the four 32-channel groups of
                                      one lane position contiguous                 */
  int32_t qk_int8; /* 0: q8/k8 hold E4M3 codes; 1: INT8 codes (QK below)          */
} absa_fp8_operands;

/* Bytes of device workspace absa_quantize_fp8 needs ([host] pointers).
 * Passage: VC-Attention page, section "İki darboğaz". */
absa_status absa_fp8_workspace(const absa_problem* prob, size_t* bytes);

/* Quantises bf16 Q, K, V ([B,H,L,128]) into `out` ([host] struct, device
 * arrays) by the rules above.  workspace: at least absa_fp8_workspace() bytes,
 * 256-byte aligned, contents on entry ignored.  Returns ABSA_ERR_UNSUPPORTED
 * unless d = 128 and Bk = 16.  Passage: VC-Attention page, section "İki
 * darboğaz" (the value term's error, the per-block mean of V removed before
 * quantising). */
absa_status absa_quantize_fp8(const absa_problem* prob, const void* q, const void* k, const void* v,
                              const absa_fp8_operands* out, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Block-sparse attention on the quantised operands: the estimate above over
 * the blocks listed for each row (same list format as absa_attend); with
 * lists == NULL every key is kept with weight 1 (dense attention in FP8).
 * o as for absa_attend.  Returns ABSA_ERR_UNSUPPORTED unless d = 128,
 * Bq = 128 and Bk = 16.  Passages: VC-Attention page, section "İki darboğaz"
 * (probabilities written as E4M3 bytes by one fused multiply-add) and section
 * "Ölçümler" (composes with sparse attention). */
absa_status absa_attend_fp8(const absa_problem* prob, const absa_fp8_operands* ops,
                            const absa_blocklist* lists, void* o, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ABSA_H_ */
