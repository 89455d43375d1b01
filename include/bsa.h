/*
 * bsa.h -- block-sparse video-DiT attention on AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The library computes one path, stage by stage:
 *   cluster layout -> centroids -> antidiagonal block scores -> per-row top-p block mask
 *   -> block-sparse flash attention with centroid compensation (or hard drop)
 *   -> exact dense probe rows -> weighted ridge fit -> correction of every row.
 *
 * Sources (cited by page title and section):
 *   [SBC] "Sparse-block compensation" (mlx-arsenal research note)
 *   [HMR] "Dynamic block masks and head-wise mask reuse" (mlx-arsenal research note)
 *   [SPR] "Partition the Support, Reconstruct the Residual" (paper summary page)
 *   [BSA] "Block-sparse attention" (topic page of paper cards), the SVG-EAR card
 *
 * Conventions shared by every call
 * --------------------------------
 * Tensors.  Q is [B, Hq, S, D]; K and V are [B, Hkv, S, D]; O has Q's shape.  All are
 *   dense row-major (the innermost dimension D is contiguous) and hold `dtype`
 *   elements (BSA_F32 = float, BSA_BF16 = bfloat16 bit patterns).  Hq must be a multiple
 *   of Hkv; query head h reads K/V head h / (Hq / Hkv) (grouped-query attention).
 *   D must be 64 or 128.
 * Labels.  Cluster labels are int32 [S] in [0, C), shared by every batch entry and head
 *   ([SBC] "Deviations from the papers": clusters are caller inputs).  A cluster layout
 *   (perm, offsets) lists token positions cluster by cluster: cluster c owns
 *   perm[offsets[c] .. offsets[c+1]).
 * Block masks.  keep is uint8 [B, Hm, Cq, Ck] (nonzero = block kept), with Hm one of
 *   1 (shared by all heads), Hkv (shared by the query heads of a K/V group, [SPR]
 *   grouped-query sharing) or Hq.  The kept-block list of a mask row is kv_count int32
 *   [B, Hm, Cq] and kv_idx int16 [B, Hm, Cq, Ck]: row r lists its kept key clusters in
 *   ascending order in kv_idx[r][0 .. kv_count[r]); the rest of the row is unused.
 * Memory.  Every pointer argument is caller-owned.  Pointers named "host" point to host
 *   memory; all others are device pointers on the current HIP device.  The library never
 *   allocates result memory; calls that need scratch memory take a caller-provided
 *   workspace of at least the size the matching *_workspace_size call reports.
 * Streams.  Device calls are asynchronous and ordered on the given stream (0 = the null
 *   stream).  They keep no state between calls and may be called from several threads.
 * Errors.  Every call validates its scalar arguments and pointers on the host before any
 *   launch; an invalid call returns an error and enqueues nothing.  BSA_E_HIP reports a
 *   failed launch (hipGetLastError).  Device-side data (labels, kv lists) is not checked:
 *   out-of-range values are skipped by the kernels rather than read or written out of
 *   bounds, and they make the result undefined.  No C++ exception crosses this ABI.
 */
#ifndef BSA_H
#define BSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BSA_OK = 0,
  BSA_E_ARG = 1,         /* null pointer or scalar out of range */
  BSA_E_SHAPE = 2,       /* sizes inconsistent with each other */
  BSA_E_DTYPE = 3,       /* unknown element type */
  BSA_E_UNSUPPORTED = 4, /* valid request this library does not implement (e.g. D = 96) */
  BSA_E_WORKSPACE = 5,   /* workspace missing or too small */
  BSA_E_HIP = 6          /* a kernel launch failed */
} bsa_status;

typedef enum { BSA_F32 = 0, BSA_BF16 = 1 } bsa_dtype;

/* Text for a status code (static storage). */
const char* bsa_status_string(int status);

/* ABI version of this header (incremented on any signature change). */
int bsa_abi_version(void);

/* ------------------------------------------------------------------------------------
 * Cluster layout.  [SPR] group-major permutation: tokens are ordered cluster by cluster,
 * keeping their given order inside a cluster (a stable counting sort of the labels).  P
 * independent layouts at once (P = 1 for one labelling of the sequence; P = B * Hkv for the
 * per-(batch, K/V head) partitions of bsa_response_partition, [SPR] grouped-query sharing).
 *   labels  int32 [P, S] in [0, C)         (tokens with other labels are left out)
 *   perm    int32 [P, S]   out: token positions in cluster-major order
 *   offsets int32 [P, C+1] out: exclusive prefix sum of counts
 *   counts  int32 [P, C]   out: tokens per cluster
 * Needs S >= 1, 1 <= C <= 8192, P <= 65535 and workspace of bsa_cluster_layout_workspace_size
 * bytes.
 *
 * Layout counts.  The calls below that read cluster layouts take n_layouts: 1 when every
 * (batch, head) shares one query layout and one key layout (arrays as above with P = 1), or
 * B * Hkv when each (batch, K/V head) has its own (layout b * Hkv + kvh, shared by that K/V
 * head's query heads; arrays [B * Hkv, ...]).  Any other value is BSA_E_ARG.
 */
bsa_status bsa_cluster_layout_workspace_size(int P, int S, int C, size_t* bytes_host);
bsa_status bsa_cluster_layout(int P, const int32_t* labels, int S, int C, int32_t* perm, int32_t* offsets,
                              int32_t* counts, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Centroids.  [SBC] "SVG-EAR -- centroid compensation": kbar_c and vbar_c are the means of
 * the keys and values of key cluster c, per (batch, K/V head); n_c = offsets[c+1]-offsets[c].
 *   K, V   [B, Hkv, S, D] dtype;  perm/offsets: key cluster layout with C clusters
 *   Kbar, Vbar float [B, Hkv, C, D] out (float32 sums; an empty cluster gives zeros)
 */
bsa_status bsa_centroids(int B, int Hkv, int S, int D, int dtype, const void* K, const void* V,
                         const int32_t* perm, const int32_t* offsets, int C, float* Kbar, float* Vbar,
                         hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Key/value packing, fused with the centroids.  [SPR] (summary page): keys and values are
 * permuted into group-major order before the sparse kernel; [SBC] "SVG-EAR -- centroid
 * compensation": kbar_c, vbar_c and n_c as for bsa_centroids.  One pass over K and V writes
 * every key cluster's keys in tiles of 64 (a cluster's last tile zero-filled) in the form
 * bsa_sparse_attention copies into on-chip memory, then the centroid tiles:
 *   K tile    [64 keys][D]  dtype
 *   V^T tile  [D][64 keys]  (keys of each 16-key group stored in the order 0-3, 8-11, 4-7,
 *             12-15) float32 inputs: float32.  bfloat16 inputs: float16 when every
 *             value of the tile is below 2^16 in magnitude and some is at least 2^-8, else
 *             bfloat16 (a per-tile flag records which, and a per-head word whether any
 *             tile of the head is bfloat16)
 * plus the first tile of every cluster.  The buffer is opaque to callers: its size comes
 * from bsa_kv_pack_workspace_size, it is valid for the key layouts (perm, offsets, C,
 * n_layouts) it was packed with, and the calls that read it must be given the same offsets
 * and n_layouts.
 *   K, V [B, Hkv, S, D] dtype;  perm int32 [n_layouts, S], offsets int32 [n_layouts, C+1]:
 *   key cluster layouts (n_layouts 1 or B * Hkv, see "Layout counts")
 *   Kbar, Vbar float [B, Hkv, C, D] out (cluster means; an empty cluster gives zeros)
 *   packed: device buffer of at least bsa_kv_pack_workspace_size bytes, packed_bytes its size
 * Needs D in {64, 128}, 1 <= C <= 32767, B * Hkv <= 65535.  BSA_E_WORKSPACE if the buffer
 * is missing or too small.
 */
bsa_status bsa_kv_pack_workspace_size(int B, int Hkv, int S, int D, int dtype, int C, int n_layouts,
                                      size_t* bytes_host);
bsa_status bsa_kv_pack(int B, int Hkv, int S, int D, int dtype, const void* K, const void* V, const int32_t* perm,
                       const int32_t* offsets, int C, int n_layouts, float* Kbar, float* Vbar, void* packed,
                       size_t packed_bytes, hipStream_t stream);
/* The same packing with caller-given centroids and counts ([SBC] API table: the compensated
 * attention takes the keys, values and clusters from the caller; "SVG-EAR -- centroid
 * compensation": column c carries log n_c and v_bar_c).  Only the token tiles are packed from
 * K and V; the centroid tiles come from Kbar/Vbar (read only), and centroid column c is
 * weighted by log(counts[c]) (a count of 0 removes the column).
 *   Kbar, Vbar float [B, Hkv, C, D]; counts int32 [n_layouts, C] (>= 0, one row per layout)
 * Other arguments, requirements and errors as bsa_kv_pack. */
bsa_status bsa_kv_pack_centroids(int B, int Hkv, int S, int D, int dtype, const void* K, const void* V,
                                 const int32_t* perm, const int32_t* offsets, int C, int n_layouts, const float* Kbar,
                                 const float* Vbar, const int32_t* counts, void* packed, size_t packed_bytes,
                                 hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Antidiagonal block scores.  [HMR] "XAttention -- anti-diagonal block scoring": over the
 * cluster-major token order (perm; NULL = identity), zero-padded to Sp = nb*block tokens
 * with nb = ceil(S / block) ([HMR] "Out of scope, and why": padding, padded keys take
 * mass), the strided logit of strided rows (i', j') is
 *     score_scale * sum_{t<stride} q[i'*stride + stride-1-t] . k[j'*stride + t],
 * each strided row is softmaxed over all Sp/stride columns, block x block tiles are summed,
 * and each row of block sums is divided by its total ([HMR] "Deviations from the papers").
 * With pool_gqa = 1 the scores of the query heads of each K/V group are averaged (the
 * group shares one mask, [SPR] grouped-query sharing).
 *   Q [B, Hq, S, D], K [B, Hkv, S, D] dtype; perm int32 [S] or NULL
 *   scores float [B, Hs, nb, nb] out, Hs = pool_gqa ? Hkv : Hq
 * Needs stride in {4, 8, 16, 32}, block % stride == 0, block / stride in {2, 4, 8, 16},
 * D in {64, 128}, and workspace of bsa_antidiag_scores_workspace_size bytes.
 */
bsa_status bsa_antidiag_scores_workspace_size(int B, int Hq, int Hkv, int S, int D, int block, int stride,
                                              size_t* bytes_host);
bsa_status bsa_antidiag_scores(int B, int Hq, int Hkv, int S, int D, int dtype, const void* Q, const void* K,
                               const int32_t* perm, int block, int stride, float score_scale, int pool_gqa,
                               float* scores, void* workspace, size_t workspace_bytes, hipStream_t stream);
/* The same scores for selected score heads only ([HMR] "HEART -- head-wise temporal mask reuse":
 * a head that keeps its mask skips the predictor).  heads: uint8 [B, Hs], nonzero = score this
 * head; rows of the other heads are left untouched in `scores` (and in the workspace).
 * BSA_E_ARG when heads is NULL; otherwise as bsa_antidiag_scores. */
bsa_status bsa_antidiag_scores_heads(int B, int Hq, int Hkv, int S, int D, int dtype, const void* Q, const void* K,
                                     const int32_t* perm, int block, int stride, float score_scale, int pool_gqa,
                                     const uint8_t* heads, float* scores, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Per-row top-p block mask.  [HMR] "XAttention -- anti-diagonal block scoring": each row
 * keeps the smallest set of key blocks whose mass reaches tau of the row total (blocks
 * taken by descending score, equal scores by lower index); [HMR] "Deviations from the
 * papers": at least one block per row, block 0 not forced.
 *   scores float [G, Cq, Ck] with G = B * Hs row groups (one per batch entry and mask head)
 *   tau    float [n_tau]: n_tau == 1 (one value) or n_tau == Hs (row group g uses tau[g % Hs])
 *   keep   uint8 [G, Cq, Ck] out;  kv_count int32 [G, Cq] out;  kv_idx int16 [G, Cq, Ck] out
 * Needs 1 <= Ck <= 1024 and 0 < tau <= 1.
 */
bsa_status bsa_top_p_mask(const float* scores, int G, int Cq, int Ck, const float* tau, int n_tau, int Hs,
                          uint8_t* keep, int32_t* kv_count, int16_t* kv_idx, hipStream_t stream);

/* Kept-block lists of a caller-given mask: keep uint8 [rows, Ck] -> kv_count int32 [rows],
 * kv_idx int16 [rows, Ck] (ascending).  Needs 1 <= Ck <= 32767. */
bsa_status bsa_mask_lists(const uint8_t* keep, int rows, int Ck, int32_t* kv_count, int16_t* kv_idx,
                          hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Block-sparse attention with centroid compensation.  [SBC] "The problem", "SVG-EAR --
 * centroid compensation" and "No LSE needed": query row i of cluster a attends to every
 * key of every kept key cluster (kv list of its mask row) and, with compensate != 0, to one
 * extra column per skipped non-empty key cluster c with logit q_i . kbar_c * scale + log n_c
 * and value vbar_c, all inside one softmax.  With compensate == 0 skipped blocks are dropped
 * (hard drop; the softmax renormalizes over kept keys).  A row with no column at all gets
 * O = 0 and lse = -inf.  Keys, values, centroids and the centroid counts are read from the
 * buffer bsa_kv_pack (or bsa_kv_pack_centroids) wrote.  out_dtype is dtype, or BSA_F32 to keep
 * the rows in float32 for a later correction (bsa_correct).
 * Repair epilogue ([SPR] Probe-Fitted Residual Reconstruction: the fitted correction applies
 * to every row): with A and c given, every row o becomes o + o A + c before it is rounded
 * once to out_dtype (o A with float32 accuracy: bfloat16 high and low parts of both operands
 * for bfloat16 inputs).  A float [B, Hq, D, D] (row-major, correction_j = sum_i o_i A[i][j]),
 * c float [B, Hq, D], both from bsa_probe_fit; NULL, NULL for no epilogue (one of them NULL:
 * BSA_E_ARG).  With A given out_dtype must equal dtype (else BSA_E_UNSUPPORTED).
 *   Q [B, Hq, S, D] dtype, O [B, Hq, S, D] out_dtype out
 *   q_perm/q_offsets (Cq clusters): query cluster layouts; k_offsets [n_layouts, Ck+1]: the key
 *     layouts the buffer was packed with; n_layouts 1 or B * Hkv ("Layout counts"; with
 *     B * Hkv > 1 layouts Hm must be Hkv or Hq, else BSA_E_SHAPE)
 *   keep/kv_count/kv_idx: block mask with Hm in {1, Hkv, Hq}
 *   packed, packed_bytes: the bsa_kv_pack buffer (BSA_E_WORKSPACE if smaller than its size)
 *   lse float [B, Hq, S] out (natural log of the softmax denominator) or NULL
 *   ws: workspace of bsa_sparse_attention_workspace_size bytes (each mask row's tile list, each
 *       K/V group's total work and the rank of each (batch, head, query cluster) unit in its
 *       group, the order in which workgroups take the units, longest first, and the staged
 *       correction of each (batch, query head))
 * Needs Ck <= 32767.  BSA_E_WORKSPACE if the packed buffer or the workspace is too small.
 */
bsa_status bsa_sparse_attention_workspace_size(int B, int Hq, int Hm, int Cq, int S, int Ck, size_t* bytes_host);
bsa_status bsa_sparse_attention(int B, int Hq, int Hkv, int S, int D, int dtype, const void* Q, float scale,
                                const int32_t* q_perm, const int32_t* q_offsets, int Cq, const int32_t* k_offsets,
                                int Ck, int n_layouts, const uint8_t* keep, const int32_t* kv_count,
                                const int16_t* kv_idx, int Hm, const void* packed, size_t packed_bytes, int compensate,
                                const float* A, const float* c, int out_dtype, void* O, float* lse, void* ws,
                                size_t ws_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): bsa_sparse_attention without a workspace
 * argument.  Its scratch memory is a static device array of
 * bsa_sparse_attention_static_scratch_bytes() bytes (48 MiB) that every GPU the library runs on
 * holds until the process ends; the call allocates nothing.  Arguments, results and errors are
 * those of bsa_sparse_attention, plus BSA_E_WORKSPACE when the problem needs more scratch than
 * the static array holds (bsa_sparse_attention_workspace_size tells) and BSA_E_HIP when the
 * array's device address cannot be obtained.  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (on different streams, or from several threads without
 * ordering) race and give undefined results; calls ordered on one stream are safe. */
size_t bsa_sparse_attention_static_scratch_bytes(void);
bsa_status bsa_sparse_attention_noalloc(int B, int Hq, int Hkv, int S, int D, int dtype, const void* Q, float scale,
                                        const int32_t* q_perm, const int32_t* q_offsets, int Cq,
                                        const int32_t* k_offsets, int Ck, int n_layouts, const uint8_t* keep,
                                        const int32_t* kv_count, const int16_t* kv_idx, int Hm, const void* packed,
                                        size_t packed_bytes, int compensate, const float* A, const float* c,
                                        int out_dtype, void* O, float* lse, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Probe rows.  [SPR] Probe-Fitted Residual Reconstruction: M query rows per (batch, head)
 * get exact dense attention over all S keys, O_dense[p] = softmax(q_p K^T scale) V ([SBC]
 * "Recipe: STA with both repairs" computes them the same way).  When O_sparse_probe is given
 * the same rows are also computed under the block-sparse rule of bsa_sparse_attention
 * (their cluster's kept blocks, plus centroid columns when Kbar/Vbar are given), in float32,
 * so the fit sees unrounded sparse outputs.
 *   probe_idx int32 [M] token positions (shared by all heads, [SBC] API table)
 *   q_labels, k_labels int32 [S]: query / key cluster labels (the layouts' labels)
 *   keep [B, Hm, Cq, Ck], k_offsets [Ck+1], Kbar/Vbar: as for bsa_sparse_attention
 *   O_dense_probe, O_sparse_probe float [B, Hq, M, D] out (O_sparse_probe may be NULL: then
 *   the label, mask and centroid arguments are ignored)
 * Needs 1 <= M <= 1024, Ck <= 2048 and workspace of bsa_probe_attention_workspace_size bytes.
 */
bsa_status bsa_probe_attention_workspace_size(int B, int Hq, int S, int D, int M, size_t* bytes_host);
bsa_status bsa_probe_attention(int B, int Hq, int Hkv, int S, int D, int dtype, const void* Q, const void* K,
                               const void* V, float scale, const int32_t* probe_idx, int M, const int32_t* q_labels,
                               const int32_t* k_labels, const uint8_t* keep, int Hm, int Cq, int Ck,
                               const int32_t* k_offsets, const float* Kbar, const float* Vbar, float* O_dense_probe,
                               float* O_sparse_probe, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The probe rows of bsa_probe_attention from the packed K/V buffer of bsa_kv_pack (bfloat16
 * inputs), in one pass over the packed tiles: the dense rows with the keys visited in the
 * packed cluster-major order (the softmax over all keys does not depend on it), and, when
 * O_sparse_probe is given, the same probes under the block-sparse rule of
 * bsa_sparse_attention (the kept key clusters of each probe's query cluster, plus, with
 * compensate != 0, the centroid columns of its skipped clusters, weighted by the pack's
 * counts), both in float32 -- the inputs of bsa_probe_fit, available before the attention runs.
 * packed, packed_bytes: the bsa_kv_pack buffer made from the same K, V and key layouts;
 * k_offsets int32 [n_layouts, C+1], C and n_layouts: those layouts' cluster offsets, cluster
 * count (C = Ck) and number ("Layout counts").  With n_layouts = B * Hkv each layout has its
 * own probes: probe_idx int32 [n_layouts, M] (else [M], shared by every head).
 *   q_labels int32 [n_layouts, S]: query cluster labels; keep uint8 [B, Hm, Cq, C]: the block
 *     mask (Hm in {1, Hkv, Hq}); both ignored when O_sparse_probe is NULL
 *   O_dense_probe, O_sparse_probe float [B, Hq, M, D] out (O_sparse_probe may be NULL)
 * Needs dtype BSA_BF16 (BSA_E_UNSUPPORTED for float32: use bsa_probe_attention), 1 <= M <= 1024,
 * C <= 1024 for sparse rows, and workspace of bsa_probe_attention_packed_workspace_size bytes.
 */
bsa_status bsa_probe_attention_packed_workspace_size(int B, int Hq, int Hkv, int S, int D, int M, int C,
                                                     size_t* bytes_host);
bsa_status bsa_probe_attention_packed(int B, int Hq, int Hkv, int S, int D, int dtype, const void* Q, float scale,
                                      const int32_t* probe_idx, int M, const void* packed, size_t packed_bytes,
                                      const int32_t* k_offsets, int C, int n_layouts, const int32_t* q_labels,
                                      const uint8_t* keep, int Hm, int Cq, int compensate, float* O_dense_probe,
                                      float* O_sparse_probe, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Ridge fit.  [SPR] Probe-Fitted Residual Reconstruction and [SBC] "Deviations from the
 * papers".  Per (batch, head), from the sparse rows X0 = O_sparse_probe and the exact rows
 * O_dense_probe of the M probes:
 *   w = weights / sum(weights); R = O_dense_probe - X0;
 *   mu = sum w X0; sigma = sqrt(sum w (X0 - mu)^2) (below 1e-6 -> 1); X = (X0 - mu) / sigma;
 *   rbar = sum w R; Rc = R - rbar;  W = (X^T W X + lambda I)^-1 X^T W Rc   (W = diag(w));
 *   P = V_r V_r^T with V_r the top min(rank, #eigenvalues > 1e-12 * max) eigenvectors of
 *   Rc^T diag(w) Rc;  A = diag(1/sigma) W P;  c = rbar - mu A.
 * The correction of any row o is then o A + c.  Computed in float64 on the device.
 *   O_sparse_probe, O_dense_probe float [B, Hq, M, D]; weights float [n_layouts, M] > 0 (n_layouts
 *   1: one set for every head; B * Hkv: head (b, h) takes row b * Hkv + h / (Hq / Hkv), the
 *   weights of its layout's probes)
 *   A float [B, Hq, D, D] out (row-major: correction_j = sum_i o_i A[i][j] + c_j); c float [B, Hq, D] out
 * Needs 2 <= M <= 65536, lambda > 0 and 1 <= rank <= 16 (rank <= D).  Up to 64 probes the fit
 * runs in its M x M dual form (the probe rows held in LDS); with more, in the D x D primal form,
 * the probe rows streamed from global memory.  Both give the map above.
 */
bsa_status bsa_probe_fit(int B, int Hq, int Hkv, int D, const float* O_sparse_probe, const float* O_dense_probe,
                         const float* weights, int M, int n_layouts, float lambda, int rank, float* A, float* c,
                         hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Correction of every row ([SPR]: the correction is applied to all rows; probe rows are
 * corrected too, not overwritten), per (batch, head).
 * bsa_correct: O_out = O_in + O_in A + c from float32 rows O_in [B, Hq, S, D] (the attention
 *   output kept in float32), rounded once to out_dtype; O_out [B, Hq, S, D] out_dtype.  For
 *   bfloat16 output the product O_in A is taken with both operands split into high and low
 *   bfloat16 parts (float32 accuracy).  With out_dtype BSA_F32, O_out may be O_in.
 * bsa_probe_apply: O <- O + O A + c, in place, for outputs already rounded to dtype.
 */
bsa_status bsa_correct(int B, int Hq, int S, int D, int out_dtype, const float* O_in, const float* A,
                       const float* c, void* O_out, hipStream_t stream);
bsa_status bsa_probe_apply(int B, int Hq, int S, int D, int dtype, void* O, const float* A, const float* c,
                           hipStream_t stream);

/* Rows of float32 outputs at given positions: out [BH, M, D] = X [BH, S, D] at rows idx [M]
 * (the probe rows of the uncorrected attention output, for bsa_probe_fit).  Indices outside
 * [0, S) leave their output row untouched. */
bsa_status bsa_gather_rows(int BH, int S, int D, const float* X, const int32_t* idx, int M, float* out,
                           hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Head-wise temporal mask reuse.  [HMR] "HEART -- head-wise temporal mask reuse" (Temporal
 * Mask Reuse), "What mlx-arsenal ships" (pooled summary, L1 drift, two-phase cache with an
 * optional layer gate), "Recipe" (the first call refreshes every head), "Deviations from the
 * papers" (relative drift).  A step is: bsa_pooled_qk, bsa_mask_reuse_decide, then the
 * predictor for the refreshed heads (bsa_antidiag_scores_heads + bsa_top_p_mask into fresh
 * mask buffers), then bsa_mask_reuse_update; attention then reads the cached mask.  The cache
 * (anchors and mask) is caller-owned device memory; calls only touch the rows of heads
 * whose refresh flag is set.
 *
 * bsa_pooled_qk: the summary of each mask head, the token mean of the queries and keys its
 * mask serves: Hm == Hq: query head m and its K/V head; Hm == Hkv: the group's query heads
 * and its K/V head; Hm == 1: all heads.  Float32 sums in a fixed order.
 *   Q [B, Hq, S, D], K [B, Hkv, S, D] dtype;  qbar, kbar float [B, Hm, D] out
 *   workspace: bsa_pooled_qk_workspace_size bytes (per-chunk partial sums)
 * Needs D in {64, 128}, Hq % Hkv == 0, Hm in {Hq, Hkv, 1}.
 */
bsa_status bsa_pooled_qk_workspace_size(int B, int Hq, int Hkv, int S, int D, size_t* bytes_host);
bsa_status bsa_pooled_qk(int B, int Hq, int Hkv, int S, int D, int dtype, const void* Q, const void* K, int Hm,
                         float* qbar, float* kbar, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* bsa_mask_reuse_decide: drift[b, m] = ||qbar - anchor_q||_1 + ||kbar - anchor_k||_1 over D
 * (relative = 1: divided by ||anchor_q||_1 + ||anchor_k||_1; a zero anchor norm gives 0 if
 * nothing moved, +inf otherwise), in float32.  A head asks for a refresh when drift > delta.
 * gate = 1 applies the layer override per batch entry over its Hm heads: fewer than 40%
 * asking -> no head refreshes, more than 80% -> every head; otherwise each head's own request.
 * have_anchor = 0 (the first call; anchors may be NULL): every head refreshes, drift = 0.
 *   qbar, kbar, anchor_q, anchor_k float [B, Hm, D]
 *   drift float [B, Hm] out (or NULL);  refresh uint8 [B, Hm] out (1 = rebuild the mask)
 * BSA_E_ARG for flags outside {0, 1}, a NaN delta or missing pointers.
 */
bsa_status bsa_mask_reuse_decide(int B, int Hm, int D, const float* qbar, const float* kbar, const float* anchor_q,
                                 const float* anchor_k, int have_anchor, float delta, int relative, int gate,
                                 float* drift, uint8_t* refresh, hipStream_t stream);

/* bsa_mask_reuse_update: for every (b, m) with refresh[b, m] != 0, copy that head's rows of
 * the new mask into the cached mask and move its anchor to the current summary; other heads
 * are untouched.  With new_keep == NULL only the anchors move (new_count and new_idx must be
 * NULL too; the cached mask pointers may then be NULL).
 *   refresh uint8 [B, Hm];  qbar, kbar float [B, Hm, D];  anchor_q, anchor_k float [B, Hm, D] in/out
 *   new_keep uint8 [B, Hm, Cq, Ck], new_count int32 [B, Hm, Cq], new_idx int16 [B, Hm, Cq, Ck]
 *   keep, kv_count, kv_idx: the cached mask, same layouts, in/out
 */
bsa_status bsa_mask_reuse_update(int B, int Hm, int Cq, int Ck, int D, const uint8_t* refresh, const float* qbar,
                                 const float* kbar, const uint8_t* new_keep, const int32_t* new_count,
                                 const int16_t* new_idx, uint8_t* keep, int32_t* kv_count, int16_t* kv_idx,
                                 float* anchor_q, float* anchor_k, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Error-aware routing.  [BSA] SVG-EAR card: centroid compensation fails on a few blocks;
 * a light probe estimates every block's compensation error and the blocks with the highest
 * error-to-cost ratio are computed exactly, the rest compensated ([SBC] "SVG-EAR --
 * centroid compensation" and "Out of scope, and why": a routing policy on top of the
 * compensated attention).  Three calls, in order: the probes, the block errors, the routes;
 * the routes are a block mask (Hm = Hq) for bsa_sparse_attention.
 *
 * bsa_query_centroids: the probe of query cluster a is its mean query row, rounded to dtype
 * (as the centroid keys are); an empty cluster gets a zero row.  Float32 sums.
 *   Q [B, Hq, S, D] dtype; q_perm/q_offsets: the query cluster layouts (Cq clusters,
 *   n_layouts 1 or B * Hkv: "Layout counts"); qbar [B, Hq, Cq, D] dtype out
 */
bsa_status bsa_query_centroids(int B, int Hq, int Hkv, int S, int D, int dtype, const void* Q, const int32_t* q_perm,
                               const int32_t* q_offsets, int Cq, int n_layouts, void* qbar, hipStream_t stream);

/* bsa_block_error: for probe q = qbar[b, h, a] with softmax weights p_j over all keys, dense
 * output O_a, and for key cluster c (n_c keys, means k_bar_c, v_bar_c from bsa_kv_pack):
 * N_c = sum_{j in c} p_j v_j, Z_c = sum_{j in c} p_j, z_hat = exp(q . k_bar_c * scale +
 * log n_c - lse_a), err[b, h, a, c] = || z_hat v_bar_c - N_c - O_a (z_hat - Z_c) ||_2, the
 * first-order change of the probe's output when block (a, c) alone is compensated; 0 for
 * an empty cluster.  Two passes over the packed tiles: the probes' dense rows and
 * log-sum-exp, then the per-cluster sums (P V with P split into two float16 parts).
 *   qbar [B, Hq, Cq, D] bfloat16; packed/packed_bytes, k_offsets [n_layouts, Ck+1], n_layouts,
 *   Kbar/Vbar float [B, Hkv, Ck, D]: the bsa_kv_pack buffer, its layouts and centroids;
 *   err float [B, Hq, Cq, Ck] out
 *   ws: workspace of bsa_block_error_workspace_size bytes (the first pass's partial rows,
 *       its rows and log-sum-exp)
 * bfloat16 only (BSA_E_UNSUPPORTED for float32).  Needs Cq <= 4096, Ck <= 32767.
 */
bsa_status bsa_block_error_workspace_size(int B, int Hq, int Hkv, int S, int D, int Cq, int Ck, size_t* bytes_host);
bsa_status bsa_block_error(int B, int Hq, int Hkv, int S, int D, int dtype, const void* qbar, int Cq, float scale,
                           const void* packed, size_t packed_bytes, const int32_t* k_offsets, int Ck, int n_layouts,
                           const float* Kbar, const float* Vbar, float* err, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/* bsa_error_route: per mask row, the non-empty key clusters in order of err / n_c (float32,
 * correctly rounded; descending, ties by lower index -- the cost of block (a, c) is
 * n_a n_c and n_a is fixed along a row) and the shortest prefix whose key count reaches
 * `budget` tokens; at least one cluster; empty clusters are never kept.
 *   err float [rows, Ck]; keep uint8 [rows, Ck], kv_count int32 [rows], kv_idx int16 [rows, Ck]
 *   out (the bsa_top_p_mask conventions)
 *   k_offsets: the key layout [Ck+1] of every row (rows_per_layout = 0), or key layouts
 *   [rows / rows_per_layout, Ck+1], row r reading layout r / rows_per_layout (rows of
 *   [B, Hq, Cq] and per-(batch, K/V head) layouts: rows_per_layout = (Hq / Hkv) * Cq)
 * Needs Ck <= 1024; rows a multiple of rows_per_layout.
 */
bsa_status bsa_error_route(const float* err, int rows, int Ck, const int32_t* k_offsets, int rows_per_layout,
                           int budget, uint8_t* keep, int32_t* kv_count, int16_t* kv_idx, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Response-coupled partitioning.  [SPR] Response-Coupled Partitioning: queries sampled from
 * the call; keys grouped by their pre-softmax response profiles to those queries (feature
 * rank rK = 48); the key groups' centroids give the query coordinates (rank rQ = 64); one
 * asymmetric pass (keys, then queries); [SPR] grouped-query sharing: one key partition and one
 * query partition per (batch, K/V head), shared by the group's query heads; [SPR] timing: an
 * online k-means inside the call.  Readings of what the page leaves open:
 *   - the rK sampled queries are the tokens floor((j + 1/2) S / rK), j < rK, of query head
 *     kvh * G + (j mod G) (G = Hq / Hkv); a key's profile is (k . q_s) * scale over them;
 *   - a query token's coordinates are (qm . kbar_c) * scale for the key groups c =
 *     floor((j + 1/2) Ck / rQ'), j < rQ' = min(rQ, Ck), with qm the mean of its G query rows
 *     and kbar_c the mean of group c's keys, scaled to unit length (zero stays zero);
 *   - k-means: starting centres at the points floor((c + 1/2) N / C); `iters` Lloyd
 *     iterations (nearest centre by squared distance, equal distances to the lower index; a
 *     centre without points keeps its place); then a last assignment, so every label is a
 *     nearest centre of the final centres.  Distances are taken as |c|^2 - 2 x.c, with x.c from
 *     split-bfloat16 products (hi.hi + hi.lo + lo.hi, float32 sums: within about 3e-5 |x| |c|).
 *   Q [B, Hq, S, D], K [B, Hkv, S, D] dtype; 1 <= rK, rQ <= 64; 1 <= Cq, Ck <= min(8192, S)
 *   k_labels, q_labels int32 [B, Hkv, S] out: the key group of every key and the query group
 *     of every query token of each (batch, K/V head)
 *   k_centres float [B, Hkv, Ck, 64], q_centres float [B, Hkv, Cq, 64] out or NULL: the final
 *     centres (features past the rank are zero)
 *   ws: bsa_response_partition_workspace_size bytes (features, centroids, the k-means sort)
 *
 * bsa_kmeans: the k-means above on its own, for P independent problems of N points with nf <= 64
 * features, stored 64 floats per point (zero past nf).  X float [P, N, 64]; labels int32 [P, N]
 * out; centres float [P, C, 64] out; C <= min(8192, N); ws of bsa_kmeans_workspace_size bytes.
 */
bsa_status bsa_response_partition_workspace_size(int B, int Hkv, int S, int D, int Cq, int Ck, size_t* bytes_host);
bsa_status bsa_response_partition(int B, int Hq, int Hkv, int S, int D, int dtype, const void* Q, const void* K,
                                  float scale, int rK, int rQ, int Cq, int Ck, int iters, int32_t* k_labels,
                                  int32_t* q_labels, float* k_centres, float* q_centres, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);
bsa_status bsa_kmeans_workspace_size(int P, int N, int C, size_t* bytes_host);
bsa_status bsa_kmeans(int P, int N, int nf, const float* X, int C, int iters, int32_t* labels, float* centres,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Probe rows on the device, from P cluster layouts (the per-(batch, K/V head) partitions of
 * bsa_response_partition after bsa_cluster_layout): the rule of bsa_select_probe_rows below,
 * applied to each layout with its members in layout order (ascending positions).
 *   perm int32 [P, S], offsets int32 [P, C+1]; probe_idx int32 [P, M] out, weights float [P, M]
 *   out (normalized per layout).  Needs 1 <= M <= S and every layout's perm a permutation of
 *   its S tokens (labels in [0, C)).
 */
bsa_status bsa_select_probe_rows_layouts(int P, int S, int C, int M, const int32_t* perm, const int32_t* offsets,
                                         int32_t* probe_idx, float* weights, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Host helpers (host pointers only).
 *
 * Probe rows.  [SBC] API table and "Deviations from the papers": probes are shared by all
 * heads; each query cluster's members are taken middle-out (positions in ascending order,
 * member floor(n/2) first, then n/2-1, n/2+1, n/2-2, ...), round-robin over clusters; each
 * probe of cluster a weighs |G_a| / m_a (cluster size over probes taken from it) and the
 * weights are normalized to sum to 1.  When M is below the number of non-empty clusters the
 * single round visits clusters floor((j + 1/2) * C_nonempty / M), j < M, spreading the
 * probes over the sequence ([SPR]: probes are stratified across query groups).
 *   labels_host int32 [S]; probe_idx_host int32 [M] out; weights_host float [M] out
 */
bsa_status bsa_select_probe_rows(const int32_t* labels_host, int S, int C, int M, int32_t* probe_idx_host,
                                 float* weights_host);

/* Sliding-tile labels of a T x H x W raster-order grid ([SBC] API table: tile_labels).
 * chunk == 0: the id of the (tt, th, tw) tile holding each token (tiles in raster order,
 * edge tiles partial).  chunk > 0: tokens ranked tile-major (raster order inside a tile),
 * label = rank / chunk.   labels_host int32 [T*H*W] out. */
bsa_status bsa_tile_labels(int T, int H, int W, int tt, int th, int tw, int chunk, int32_t* labels_host);

/* Static sliding-tile block mask ([SBC] "Recipe: STA with both repairs": built at tile
 * resolution and used with the tile labels; expanded through them it is the token-level
 * mask).  Cells of an nT x nH x nW raster grid form tiles of (tt, th, tw) cells (edge tiles
 * partial); cell i keeps cell j when j's tile lies in the window of (wt, wh, ww) tiles around
 * i's tile.  Along an axis of n tiles the window of w tiles around coordinate a starts at
 * min(max(a - w/2, 0), max(n - w, 0)): it slides inward at the edges, so every row keeps
 * the same number of tiles.  With (tt, th, tw) = (1, 1, 1) the cells are tiles and the
 * result is the cluster-level mask for bsa_tile_labels clusters.
 *   keep_host uint8 [N, N] out, N = nT * nH * nW (at most 65535)
 */
bsa_status bsa_sliding_tile_mask(int nT, int nH, int nW, int tt, int th, int tw, int wt, int wh, int ww,
                                 uint8_t* keep_host);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H */
