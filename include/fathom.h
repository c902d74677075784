/*
 * fathom.h -- C ABI of libfathom, a gfx950 (MI355X) implementation of the
 * Fathom per-query variable-read-depth key scan over a bit-plane 4-bit K cache.
 *
 * Method pages:
 *   [Art] "Fathom Makes KV-Cache Scans Query-Adaptive for Long-Context
 *         Decoding" (paragraphs 1-3 and the limits paragraph);
 *   [Abs] "Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded
 *         KV Caches", abstract sentences s1-s6.
 * The pages state no programming interface; the arguments below follow their
 * statement of the problem (a K cache, a query, a bit budget B, a top-k k)
 * plus layout descriptors.
 *
 * Conventions shared by every entry point
 *   - Ownership: the caller owns every buffer.  The library allocates nothing
 *     inside fathom_pack_planes, fathom_allocate or fathom_scan_topk; scratch
 *     memory comes in through `workspace`, sized by fathom_workspace_bytes.
 *   - Pointers are device pointers (HBM), except `planes` in fathom_scan_topk,
 *     which may also be the device view of pinned host memory obtained from
 *     fathom_host_device_pointer (zero-copy reads over PCIe).
 *   - Asynchrony: work is enqueued on `hip_stream` (a hipStream_t passed as
 *     void*, NULL = the legacy default stream).  Outputs are valid once the
 *     stream has been synchronized.
 *   - Validation happens on the host before any HIP call.  On error nothing
 *     is launched, outputs are untouched, a negative status is returned and
 *     fathom_last_error() describes the problem.  No C++ exception crosses
 *     this boundary.
 *   - Layout of the plane store ("channel-major bit planes", [Art] para 2,
 *     [Abs] s3): planes[h][c][j][w], uint32, j = 0 is the most significant
 *     bit of the 4-bit code; word w of a row holds keys 32w..32w+31 with key
 *     32w+b at bit b; rows are `ldw` words long (ldw % 4 == 0) and bits of
 *     keys >= n are zero.  A t-plane prefix of channel c is the contiguous
 *     run planes[h][c][0..t-1][*].
 *   - Query head q reads KV head q / group; num_q must equal H * group
 *     (grouped-query attention; sessions are flattened into H).
 *   - Supported: d = 128 channels, 1 <= n <= 2^26 keys per head, and one
 *     head's plane block (d * 4 * ldw words) below 4 GiB, i.e. ldw <= 2^21 - 4
 *     (the scan addresses a head with 32-bit byte offsets); larger stores are
 *     rejected with FATHOM_ERR_UNSUPPORTED.  Keys and queries must be finite.
 */
#ifndef FATHOM_H
#define FATHOM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every int-returning entry point. */
enum {
  FATHOM_OK = 0,
  FATHOM_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, bad size or range */
  FATHOM_ERR_UNSUPPORTED = -2,  /* valid but not implemented (d != 128, ...)  */
  FATHOM_ERR_WORKSPACE = -3,    /* workspace missing, misaligned or too small */
  FATHOM_ERR_HIP = -4           /* a HIP runtime call or launch failed        */
};

/* Operation selector for fathom_workspace_bytes. */
enum { FATHOM_OP_PACK = 0, FATHOM_OP_SCAN = 1, FATHOM_OP_ATTEND = 2 };

/* Control-read modes of fathom_control_allocate. */
enum { FATHOM_CONTROL_UNIFORM = 0, FATHOM_CONTROL_TOP_CHANNELS = 1 };

/* Largest k accepted by fathom_scan_topk. */
#define FATHOM_MAX_K 4096

/* Shape of a plane store: H KV heads, d channels, n keys per head, ldw words
 * per plane row.  Passed by pointer; the library does not keep it.
 *
 * lengths (ragged sessions: [Art] para 1, many sessions of different lengths
 * decode at once): NULL, or a device array int32 [H] holding the number of
 * keys of each head.  Head h then holds n_h = min(max(lengths[h], 0), n)
 * keys, n being the bound no head exceeds (ldw >= ceil(n / 32) as always).
 * With lengths:
 *   - fathom_pack_planes quantizes each head over its own n_h keys (a head
 *     with n_h = 0 gets lo = step = var = 0 and all-zero planes);
 *   - fathom_append_keys writes head h's new keys at position n_h and adds m
 *     to lengths[h];
 *   - the scans rank head h's n_h keys only: no index >= n_h is returned, and
 *     a query whose head holds fewer than k keys gets its n_h keys followed
 *     by index -1 with score -inf;
 *   - fathom_sparse_attention skips indexes >= n_h.
 * Bits of keys >= n_h are zero after packing (appends keep them so).  The
 * array is read on the device when the work runs, so it is not validated on
 * the host; out-of-range values are clamped as above. */
typedef struct fathom_store_desc {
  int32_t num_kv_heads;
  int32_t d;
  int64_t n;
  int64_t ldw;
  int32_t* lengths;
} fathom_store_desc;

/* Words per plane row for n keys: ceil(n / 32) rounded up to a multiple of 4
 * (16-byte rows).  Returns -1 when n < 1. */
int64_t fathom_plane_ldw(int64_t n);

/* Bytes of device workspace needed by an operation (FATHOM_OP_PACK: num_q and
 * k are ignored; FATHOM_OP_SCAN: the scan + top-k of num_q queries;
 * FATHOM_OP_ATTEND: attention of num_q queries over k selected rows).  Returns
 * 0 for an invalid description.  The workspace pointer must be 256-byte
 * aligned. */
size_t fathom_workspace_bytes(int32_t op, const fathom_store_desc* store, int32_t num_q, int32_t k);

/* Quantize-and-transpose packer ([Art] para 2; [Abs] s3, s6).
 * keys: float32, key i of head h at keys[h*stride_head + i*stride_token + c]
 *   (channel stride 1; 16-byte aligned base, stride_token % 4 == 0).
 * Per (head, channel) asymmetric 4-bit floor quantizer over the head's n keys:
 *   lo = min K, r = fl32(max K - lo), step = r/16, inv = fl32(16/r) (0 if r=0),
 *   code = min(15, floor(fl32(fl32(K - lo) * inv))).
 * Writes planes [H][d][4][ldw] (all words, padding bits zero), lo [H][d],
 * step [H][d], and, if var != NULL, var [H][d] = variance of the 4-bit
 * reconstructions lo + (code + 1/2) step from exact integer moments:
 *   fl32( fl64(S2 n - S1^2) / fl64(n^2) * fl64(step)^2 ).
 * The result is bit-exact and independent of launch order.
 * workspace: >= fathom_workspace_bytes(FATHOM_OP_PACK, ...) bytes. */
int fathom_pack_planes(const float* keys, int64_t stride_head, int64_t stride_token,
                       const fathom_store_desc* store, uint32_t* planes, float* lo, float* step,
                       float* var, void* workspace, size_t workspace_bytes, void* hip_stream);

/* Decode-time append ([Abs] s1; [Art] para 1: the cache grows by a token per
 * step): keys n .. n + m - 1 of every head, with n = store->n the head's
 * current length, are written into the planes of a store packed by
 * fathom_pack_planes, under the head's packed quantizer: r = fl32(16 step),
 * inv = fl32(16 / r) (0 if r = 0), code = min(15, max(0, floor(fl32(fl32(K -
 * lo) * inv)))) -- the packer's rule, clamped since a new key may fall outside
 * the packed range.  The bits of those keys are replaced; no other bit, and
 * neither lo, step nor var, changes.  keys: float32, key n + t of head h at
 * keys[h*stride_head + t*stride_token + c] (channel stride 1); 1 <= m and
 * n + m <= 32 * store->ldw (the rows' capacity).  Afterwards the store holds
 * n + m keys: pass n + m to the scan.  One kernel launch on hip_stream.
 * With store->lengths, head h's keys go to positions n_h .. n_h + m - 1
 * (n_h as clamped there) and lengths[h] becomes n_h + m, in a second launch;
 * n + m <= 32 * ldw still bounds every head, and n + m is the new bound. */
int fathom_append_keys(const float* keys, int64_t stride_head, int64_t stride_token, int32_t m,
                       const fathom_store_desc* store, uint32_t* planes, const float* lo, const float* step,
                       void* hip_stream);

/* Per-query bit allocation by reverse water-filling ([Art] para 3; [Abs] s2,
 * s3).  q: float32 [num_q][d]; var: float32 [H][d] (any calibrated channel
 * variance, e.g. the packer's); budget_bits B in [0, 4d].
 * w_c = fl32(fl32(q_c^2) var_c); candidate (c, j) has the int32 ordering key
 * bits(w_c) - j*2^24 (the order of w_c 4^-j); the B best candidates by
 * (key desc, c asc, j asc) are taken and alloc[q][c] = number taken from c.
 * var holds variances, so >= 0: a weight w_c that is not a positive number
 * (from a negative, -0 or NaN var_c) is read as +0: the channel has no
 * importance.  The same rule holds in fathom_allocate_scan_topk.
 * Output alloc: uint8 [num_q][d], every row sums to B, entries in 0..4. */
int fathom_allocate(const float* q, int32_t num_q, int32_t group, const float* var,
                    const fathom_store_desc* store, int32_t budget_bits, uint8_t* alloc,
                    void* hip_stream);

/* Fixed-depth control allocations: the read widths the pages compare Fathom
 * with (fixed 136- and 68-bit scans; [Art] findings bullets 1-2; [Abs] s4),
 * as allocations that fathom_scan_topk reads like any other.
 * q: float32 [num_q][d] (d = 128, 8-byte aligned); budget_bits B in [0, 4d];
 * alloc: uint8 [num_q][d] (2-byte aligned).  Channels are ranked by |q_c|
 * descending, ties to the lower channel index.
 *   FATHOM_CONTROL_UNIFORM: every channel reads floor(B/d) planes, and the
 *     first B mod d channels in rank order one more.
 *   FATHOM_CONTROL_TOP_CHANNELS: the first floor(B/4) channels read all 4
 *     planes and the next one B mod 4.
 * Every row sums to B.  Returns FATHOM_ERR_INVALID_ARG for a bad mode,
 * budget, count or alignment (nothing is launched). */
int fathom_control_allocate(const float* q, int32_t num_q, int32_t mode, int32_t budget_bits, uint8_t* alloc,
                            void* hip_stream);

/* Plane-prefix scan with fused top-k ([Art] paras 1-2; [Abs] s1-s3).
 * For every query q (KV head h = q / group) and key i < n:
 *   s_q(i) = C_q + sum_c sum_{j < b_qc} q_c step_c 2^(3-j) bit_{c,j}(i),
 *   C_q = sum_c q_c (lo_c + step_c 2^(3-b_qc)),
 * which is the dot product of q with the keys dequantized from their b_qc-bit
 * prefixes at the bin centres.  Only the planes j < max over the group of
 * b_qc are read.  Outputs, per query, the k best keys by (score desc,
 * index asc): out_idx int32 [num_q][k], out_score float32 [num_q][k].
 * all_scores: NULL, or float32 [num_q][n] receiving every score (a debug and
 * parity aid; costs n*4 bytes of writes per query).
 * alloc values above 4 are read as 4.
 * Score arithmetic (fixed point, on the int8 matrix cores): per query, let U
 * be the union of its group's plane prefixes and S = sum over its planes in U
 * of |W| with W = q_c step_c 2^(3-j) (0 where the query skips the plane).
 * Each weight is rounded to the integer V = round(W 2^30 / S); the sum
 * t = sum V bit over the key's planes is exact in int32 (int8 digits of V,
 * int32 matrix-core accumulation, exact recombination), and the returned
 * score is fl32(fl32(t) * fl32(S 2^-30) + C_q) with C_q summed in float64
 * and rounded once.  Its distance from the exact real score is at most
 * (|U| / 2) 2^-30 S (weight rounding, |U| <= 512) plus the two fp32
 * roundings.  The top-k is exact over these scores.
 * workspace: >= fathom_workspace_bytes(FATHOM_OP_SCAN, store, num_q, k). */
int fathom_scan_topk(const uint32_t* planes, const float* lo, const float* step,
                     const fathom_store_desc* store, const float* q, const uint8_t* alloc,
                     int32_t num_q, int32_t group, int32_t k, int32_t* out_idx, float* out_score,
                     float* all_scores, void* workspace, size_t workspace_bytes, void* hip_stream);

/* Allocation and scan in one call: the same results as fathom_allocate
 * (budget_bits, var) followed by fathom_scan_topk with that allocation, which
 * is also written to alloc (uint8 [num_q][d]).  The allocation is computed
 * inside the scan's first kernel (one wavefront per query of each KV-head
 * chunk), so the pair costs one kernel launch less.  Arguments as in the two
 * calls; no all_scores output. */
int fathom_allocate_scan_topk(const uint32_t* planes, const float* lo, const float* step, const float* var,
                              const fathom_store_desc* store, const float* q, int32_t num_q, int32_t group,
                              int32_t budget_bits, int32_t k, uint8_t* alloc, int32_t* out_idx,
                              float* out_score, void* workspace, size_t workspace_bytes, void* hip_stream);

/* Staging modes of fathom_allocate_scan_topk_staged. */
enum { FATHOM_STAGE_COPY_ENGINE = 0, FATHOM_STAGE_GATHER = 1 };

/* The same decode step with the plane store in host memory, staged into HBM
 * head by head ([Art] para 1 and limits paragraph; [Abs] s1, s6: the index
 * lives in host memory, where avoiding transfers matters more than
 * arithmetic).  planes_host: the store (layout as always) in pinned host
 * memory (hipHostMalloc or torch pin_memory; not registered memory).
 * staging: device memory for two head blocks, >= 2 * d * 4 * ldw * 4 bytes,
 * 256-byte aligned.  workspace: >= fathom_workspace_bytes(FATHOM_OP_SCAN,
 * store, group, k) (one head's queries at a time).
 * The call launches the allocation of every query (alloc, as in
 * fathom_allocate).  Then, per KV head h, only the head's union rows -- per
 * channel c the contiguous rows j < u_c, u_c the deepest prefix any of the
 * head's queries reads -- are copied from planes_host into staging slot
 * h % 2 on copy_stream, while hip_stream scans head h - 1 from the other
 * slot; events order each scan after its copy and each copy after the last
 * scan (of this call or the previous one) that read its slot.
 *   FATHOM_STAGE_COPY_ENGINE: hipMemcpyAsync per run of union rows (runs
 *     closer than a copy's fixed cost are joined, rows between included);
 *     the union is needed on the host, so the call BLOCKS the calling thread
 *     until the allocation has been copied back.
 *   FATHOM_STAGE_GATHER: a kernel on copy_stream reads the union rows over
 *     PCIe in 16-byte loads (union computed on the device); no host wait.
 * Results equal those of fathom_allocate_scan_topk on the same store.
 * Outputs are valid once hip_stream has been synchronized; copy_stream must
 * be a stream of the same device (the same stream works, without overlap).
 * Concurrent staged calls share the library's events: serialize them. */
int fathom_allocate_scan_topk_staged(const uint32_t* planes_host, const float* lo, const float* step,
                                     const float* var, const fathom_store_desc* store, const float* q, int32_t num_q,
                                     int32_t group, int32_t budget_bits, int32_t k, uint8_t* alloc, int32_t* out_idx,
                                     float* out_score, uint32_t* staging, size_t staging_bytes, void* workspace,
                                     size_t workspace_bytes, int32_t mode, void* hip_stream, void* copy_stream);

/* For callers that cannot allocate memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same call as
 * fathom_allocate_scan_topk, with the same results, but its scratch memory
 * is a static device array of the library (FATHOM_NOALLOC_SCRATCH_BYTES per
 * GPU, held from the first such call on that GPU until the process ends)
 * instead of a caller workspace.  The call allocates nothing and takes no
 * workspace; the caller still passes every input and output.
 * Limits: num_q <= FATHOM_NOALLOC_MAX_Q (query heads per call) and
 * fathom_workspace_bytes(FATHOM_OP_SCAN, store, num_q, k) <=
 * FATHOM_NOALLOC_SCRATCH_BYTES (the 1M-key, 32-query, k = 2048 step needs
 * about 8 MiB), else FATHOM_ERR_UNSUPPORTED and nothing is launched.  Runs on the current HIP
 * device; hip_stream must belong to it.  Every call on one GPU shares that
 * GPU's array (each call rewrites what it reads), so calls that overlap in
 * time on one GPU -- on two streams, or from two threads -- race and must be
 * serialized by the caller.  The first call on a device looks up the array's
 * address (hipGetSymbolAddress) and may fail with FATHOM_ERR_HIP. */
#define FATHOM_NOALLOC_MAX_Q 64
#define FATHOM_NOALLOC_SCRATCH_BYTES (16 << 20)
int fathom_allocate_scan_topk_noalloc(const uint32_t* planes, const float* lo, const float* step, const float* var,
                                      const fathom_store_desc* store, const float* q, int32_t num_q, int32_t group,
                                      int32_t budget_bits, int32_t k, uint8_t* alloc, int32_t* out_idx,
                                      float* out_score, void* hip_stream);

/* Attention over the selected keys: the decode step after the top-k scan
 * ([Abs] title and s1; [Art] findings bullet 2 for its error measure).  For
 * query q (KV head h = q / group) and its k selected rows i = idx[q][0..k):
 *   p_i = exp(scale * q.k_i - max),  out[q] = sum_i p_i v_i / sum_i p_i,
 * accumulated in fp32.  k_rows, v_rows: bf16 (uint16 bit patterns); row i of
 * head h at [h * stride_head + i * stride_token], channel stride 1, d = 128;
 * device pointers or device-visible pinned host pointers (rows then cross
 * PCIe).  Bases 16-byte aligned, strides in elements, multiples of 8,
 * stride_token >= d.  q: float32 [num_q][d]; idx: int32 [num_q][k] (typically
 * fathom_scan_topk's out_idx; an index outside [0, n) is skipped); scale
 * finite (e.g. 1/sqrt(d)); out: float32 [num_q][d] (0 for a query with no
 * index in range).  1 <= k <= min(n, FATHOM_MAX_K).
 * workspace: >= fathom_workspace_bytes(FATHOM_OP_ATTEND, store, num_q, k)
 * bytes, 256-byte aligned.  Two kernel launches on hip_stream. */
int fathom_sparse_attention(const uint16_t* k_rows, const uint16_t* v_rows, int64_t stride_head,
                            int64_t stride_token, const fathom_store_desc* store, const float* q,
                            const int32_t* idx, int32_t num_q, int32_t group, int32_t k, float scale,
                            float* out, void* workspace, size_t workspace_bytes, void* hip_stream);

/* Device-visible address of pinned host memory (allocated with hipHostMalloc
 * or torch pin_memory), for a plane store kept in host RAM ([Art] para 1;
 * [Abs] s1: the index lives in host memory).  Not for registered memory. */
int fathom_host_device_pointer(void* pinned_host, void** device_ptr);

/* Static text for a status code. */
const char* fathom_status_string(int32_t status);

/* Detail of the last error on the calling thread ("" if none). */
const char* fathom_last_error(void);

/* Kernel timing for measurement: while enabled, the library records HIP
 * events carried by the dispatch of the main scan kernel of each
 * fathom_scan_topk call (on the call's stream).  Enabling or disabling keeps
 * the record; fathom_timing_read synchronizes on the recorded events,
 * returns the summed kernel time (ms) and the number of timed launches since
 * the last read, and clears the record.  At most 4096 launches are kept. */
int fathom_timing_enable(int32_t enable);
int fathom_timing_read(double* total_ms, int32_t* launches);

/* Measurement aid (not a step of the method): the HBM read ceiling that the
 * scan's roofline fraction is set against.  Reads `bytes` (a positive
 * multiple of 16) at src (a 16-byte aligned device pointer) once, in 16-byte
 * non-temporal loads spread over the whole GPU, and folds them into values
 * that are written to sink (uint32 [fathom_stream_read_sink_words()], device)
 * only in the improbable case that one equals a fixed constant.  One kernel
 * launch on hip_stream; time it with events on that stream. */
int fathom_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* hip_stream);
int32_t fathom_stream_read_sink_words(void);

#ifdef __cplusplus
}
#endif

#endif /* FATHOM_H */
