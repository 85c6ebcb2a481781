/*
 * lbp.h - load-balanced paged GQA decode attention for AMD Instinct MI355X
 * (gfx950).  C ABI of liblbp.so.
 *
 * The method (SGLang x HPC-Ops page, "Scheduling around live KV work";
 * vLLM x HPC-Ops page, "Solution: per-step load-balanced decode scheduler"):
 * once per decode step an assign kernel turns the live sequence lengths
 * into a task map that spreads 64-token KV tiles evenly over a fixed number
 * of persistent workgroups; for every layer a persistent attention kernel
 * drains each workgroup's bin and writes one partial output plus its
 * log-sum-exp per task descriptor, and a light combine kernel merges each
 * (KV head, request) pair's partials into the final BF16 output (or, in
 * lbp_attend_fused, the attention kernel merges them itself).
 *
 * Conventions for every function below:
 *  - Pointers named *_dev are device pointers; everything else is host
 *    memory.  The caller allocates and owns every buffer; the library keeps
 *    no per-call state and no device memory of its own, except the fixed
 *    split-buffer array of lbp_attend_noalloc.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every launching call is asynchronous on that stream, performs no
 *    host<->device copy and no synchronisation, so it can be captured into
 *    a HIP graph.
 *  - Arguments are checked on the host before anything is launched; a bad
 *    argument returns an error status and launches nothing.  Faults inside
 *    a kernel surface at the caller's next synchronisation, as for any HIP
 *    call.  No C++ exception crosses this interface.
 *  - Concurrency: the attend calls read a plan workspace but may also update
 *    counters in it (the bin ticket counter of a DYNAMIC plan with more bins
 *    than CUs, the arrival counters of lbp_attend_fused), each back at zero
 *    when the launch completes.  Calls that share a plan workspace must
 *    therefore be ordered on one stream (the layers of a step are); calls
 *    that run concurrently need their own plan workspace (lbp_plan into each)
 *    and their own split workspace.
 *
 * Fixed data layouts (all contiguous, row-major):
 *  - q        [batch][q_len][num_q_heads][128]          bf16
 *  - out      [batch][q_len][num_q_heads][128]          bf16
 *             (q_len = cfg->q_len, 1 for plain decode)
 *  - k_cache, v_cache [num_pages][num_kv_heads][64][128] bf16, or uint8
 *             OCP e4m3 codes for LBP_KV_FP8_E4M3 (page, KV head, slot, dim)
 *  - k_scale, v_scale [num_pages][num_kv_heads][64]     fp32 (FP8 only);
 *             the stored value is e4m3(code) * scale
 *  - seq_lens [batch] int32; page_table [batch][page_table_stride] int32:
 *             token t of request r lives in page page_table[r][t / 64] at
 *             slot t % 64.  Entries past a request's last page are not read.
 *  - Query head h belongs to KV head h / (num_q_heads / num_kv_heads).
 */
#ifndef LBP_H
#define LBP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LBP_VERSION 2
#define LBP_HEAD_DIM 128
#define LBP_PAGE_SIZE 64
#define LBP_MAX_GROUP 16
#define LBP_MAX_QUERY_COLUMNS 64 /* (Hq / H_kv) * q_len */
#define LBP_PLAN_MAGIC 0x4C425031u /* "LBP1" */
/* Size of the fixed device array that lbp_attend_noalloc keeps its split
 * buffer in, one per GPU the library runs on (held until the process ends). */
#define LBP_NOALLOC_SCRATCH_BYTES (32u << 20)

typedef enum lbp_status {
  LBP_OK = 0,
  LBP_ERR_INVALID_ARG = 1,         /* NULL pointer, non-positive size, ... */
  LBP_ERR_UNSUPPORTED = 2,         /* head_dim != 128, page != 64, group * q_len > 64 */
  LBP_ERR_WORKSPACE_TOO_SMALL = 3, /* a caller workspace is below the query */
  LBP_ERR_MISMATCH = 4,            /* plan info does not match the config */
  LBP_ERR_HIP = 5,                 /* the HIP runtime refused a launch/query */
  LBP_ERR_SCRATCH_LIMIT = 6        /* lbp_attend_noalloc: the split buffer the call needs is
                                      larger than LBP_NOALLOC_SCRATCH_BYTES */
} lbp_status;

typedef enum lbp_kv_dtype { LBP_KV_BF16 = 0, LBP_KV_FP8_E4M3 = 1 } lbp_kv_dtype;

/* Scheduling policies.  DYNAMIC is the method; the two static split-KV
 * policies are the comparison the SGLang x HPC-Ops page describes under
 * "Attention: load balancing for mixed-length decode" (one fixed grid over
 * KV heads, requests and splits, with a fixed split count or a fixed chunk
 * size for every request).  All three emit the same task-map format. */
typedef enum lbp_policy {
  LBP_POLICY_DYNAMIC = 0,       /* param = F, the minimum tiles per bin (0 = cfg) */
  LBP_POLICY_STATIC_SPLITS = 1, /* param = S, splits per (KV head, request) */
  LBP_POLICY_STATIC_CHUNK = 2   /* param = C, tiles per split; every pair gets
                                   ceil(max_pages_per_seq / C) bins */
} lbp_policy;

typedef struct lbp_config {
  int32_t num_q_heads;       /* Hq >= 1 */
  int32_t num_kv_heads;      /* H_kv >= 1, Hq % H_kv == 0, Hq / H_kv <= 16 */
  int32_t head_dim;          /* must be 128 */
  int32_t page_size;         /* must be 64 (one page = one 64-token tile) */
  int32_t max_batch;         /* largest batch any plan will be built for */
  int32_t max_pages_per_seq; /* page-table row capacity; lengths above
                                64 * max_pages_per_seq are clamped and flagged */
  int32_t num_workgroups;    /* W, persistent workgroups (bins); 0 = one per CU */
  int32_t min_tiles_per_bin; /* F, the minimum-work floor in tiles; 0 = 1,
                                i.e. no floor (measured fastest on small
                                batches, where a floor cuts parallelism) */
  int32_t kv_dtype;          /* lbp_kv_dtype */
  float sm_scale;            /* softmax scale, > 0 (1/sqrt(128) typically) */
  int32_t q_len;             /* query tokens per request per step (0 = 1): > 1 for
                                speculative verification, where token j of request r
                                sits at position L_r - q_len + j and attends causally
                                to KV positions <= its own; requires
                                (Hq / H_kv) * q_len <= LBP_MAX_QUERY_COLUMNS */
} lbp_config;

/* Host-side record of a built plan, filled by lbp_plan / lbp_plan_static and
 * read by the attend calls.  Plain data; copy it freely. */
typedef struct lbp_plan_info {
  uint32_t magic;            /* LBP_PLAN_MAGIC once filled */
  int32_t policy;            /* lbp_policy */
  int32_t param;             /* F, S or C as used */
  int32_t batch;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t num_bins;          /* workgroups the attention kernel launches */
  int32_t max_desc;          /* descriptor (and split-buffer slot) capacity */
  uint64_t plan_bytes;       /* bytes of the plan workspace in use */
  const int32_t* page_table_dev; /* bound page table (must outlive the plan) */
  int64_t page_table_stride; /* in int32 entries */
} lbp_plan_info;

/* Byte offsets of the task map inside a plan workspace (for readers such as
 * tests; the kernels use the same offsets).  All sections are int32:
 *   header[16]: [0] magic [1] policy [2] num_bins [3] batch [4] num_kv_heads
 *               [5] T (tiles) [6] budget (F-floored for DYNAMIC, S or C for
 *               the static policies) [7] D (descriptors) [8] U (bins with
 *               work) [9] status bits (1 = a length was clamped) [10] bin
 *               ticket counter of the attention kernel (0 between launches)
 *               [11] number of split_list entries
 *   bin_offset[num_bins + 1]  descriptors of bin b: [bin_offset[b], bin_offset[b+1])
 *   bin_first[num_bins][8]    copy of desc[bin_offset[b]], then the physical
 *                             pages of that descriptor's first two tiles (the
 *                             second is the first's when it has one tile), 0, 0
 *                             (all zeros for an empty bin), so a workgroup
 *                             reads its bin's range, first descriptor and
 *                             first pages in one round trip
 *   desc[max_desc][4]         (kv_head, request, token_begin, token_end)
 *   pair_first[H_kv * batch], pair_count[H_kv * batch]; pair p = kv_head * batch + request
 *   scratch[H_kv * batch]     assign-kernel scratch
 *   split_list[max_split][4]  (pair, pair_first, pair_count, 0) of every pair
 *                             with pair_count >= 2, in pair order; max_split =
 *                             min(H_kv * batch, num_bins - 1) for DYNAMIC (a
 *                             pair is split only across one of the U - 1
 *                             internal bin boundaries), H_kv * batch otherwise
 *   arrive[2][max_desc]       DYNAMIC only (empty otherwise): arrival counters
 *                             of the merge lbp_attend_fused performs inside
 *                             the attention kernel; zeroed by the plan and
 *                             back at zero after every completed launch */
typedef struct lbp_plan_offsets {
  uint64_t header, bin_offset, bin_first, desc, pair_first, pair_count, scratch, split_list,
      arrive, total;
} lbp_plan_offsets;

/* Arguments of lbp_prologue (all pointers are device pointers). */
typedef struct lbp_prologue_args {
  const void* qkv;             /* [batch][q_len][(Hq + 2 * H_kv) * 128] bf16: the fused
                                  QKV projection of the new tokens, query heads, then key
                                  heads, then value heads (q_len = cfg->q_len, 1 for
                                  plain decode) */
  const int32_t* seq_lens;     /* [batch] lengths including the new tokens; token j sits at
                                  position seq_lens[r] - q_len + j (< 0: skipped) */
  const int32_t* page_table;   /* [batch][page_table_stride], as for lbp_plan */
  int64_t page_table_stride;   /* in int32 entries, >= cfg->max_pages_per_seq */
  const float* q_norm_weight;  /* [128] QK-Norm weight of the query heads */
  const float* k_norm_weight;  /* [128] QK-Norm weight of the key heads */
  const float* rope_cos_sin;   /* [max_position][128] fp32: row p holds cos(p * f_i) for
                                  the 64 rotation frequencies f_i, then sin(p * f_i) */
  int32_t max_position;        /* rows of rope_cos_sin (>= 1); later positions use the last */
  float norm_eps;              /* RMSNorm epsilon (>= 0) */
  int32_t q_fp8;               /* 1: q_out receives e4m3 codes and q_scale_out one fp32
                                  scale per (request, query head); 0: q_out is bf16 */
  void* q_out;                 /* [batch][q_len][Hq][128] bf16 or uint8 */
  float* q_scale_out;          /* [batch][q_len][Hq] (q_fp8 = 1 only) */
  void* k_cache;               /* the paged caches of lbp_attend, in cfg->kv_dtype */
  void* v_cache;
  float* k_scale;              /* [num_pages][H_kv][64] (FP8 cache only) */
  float* v_scale;
} lbp_prologue_args;

/* Human-readable name of a status code (static storage). */
const char* lbp_status_string(lbp_status s);

/* LBP_VERSION of the built library. */
int32_t lbp_version(void);

/* Workspace sizes a (config, policy, param) needs at batch = max_batch.
 * plan_bytes: the task map; split_bytes: the partial-output buffer
 * (max_desc x C x 128 fp32 plus max_desc x C fp32 log-sum-exp, with
 * C = G * q_len query rows per KV head).  Host only;
 * may query the current device's CU count when num_workgroups == 0. */
lbp_status lbp_query_workspace(const lbp_config* cfg, int32_t policy, int32_t param,
                               size_t* plan_bytes, size_t* split_bytes);

/* Dynamic plan (the method's assign step; SGLang x HPC-Ops page, "Scheduling
 * around live KV work"; vLLM x HPC-Ops page, bullet "Assign"): cut each of
 * the num_kv_heads x batch (KV head, request) pairs into ceil(L / 64) tiles,
 * set budget = max(ceil(T / W), F) from the total T, and fill bins 0..W-1 in
 * head-major, batch-minor order, each up to the budget before spilling into
 * the next; one descriptor per run of one pair in one bin.  Runs one
 * workgroup on `stream`, reading seq_lens_dev on the device (no D2H).  The
 * map is valid for every layer of the step while page_table_dev and the
 * lengths stay unchanged.  Negative lengths count as 0. */
lbp_status lbp_plan(const lbp_config* cfg, const int32_t* seq_lens_dev, int32_t batch,
                    const int32_t* page_table_dev, int64_t page_table_stride,
                    void* plan_ws_dev, size_t plan_ws_bytes, lbp_plan_info* info,
                    void* stream);

/* Static split-KV plan in the same format (comparison schedules).
 * policy = LBP_POLICY_STATIC_SPLITS: pair p's n tiles are cut into S ranges
 * of ceil(n / S) tiles, range s in bin p * S + s (empty ranges: no
 * descriptor).  policy = LBP_POLICY_STATIC_CHUNK: range s = tiles
 * [s*C, min((s+1)*C, n)) in bin p * ceil(max_pages_per_seq / C) + s. */
lbp_status lbp_plan_static(const lbp_config* cfg, int32_t policy, int32_t param,
                           const int32_t* seq_lens_dev, int32_t batch,
                           const int32_t* page_table_dev, int64_t page_table_stride,
                           void* plan_ws_dev, size_t plan_ws_bytes, lbp_plan_info* info,
                           void* stream);

/* Offsets of the task-map sections for a filled plan info (host only). */
lbp_status lbp_plan_layout(const lbp_plan_info* info, lbp_plan_offsets* offsets);

/* Copies a plan's task map (the first lbp_plan_layout(info).total bytes of
 * plan_ws_dev, laid out as lbp_plan_offsets describes) into host_buf, in
 * order after the work already on `stream`, and waits for the copy: for
 * tests and inspection of what the assign step built (SGLang x HPC-Ops
 * page, "Scheduling around live KV work"), never for the decode path.  The
 * only call in the library that synchronises.  host_buf (caller-owned, any
 * host memory) must hold host_bytes >= that total, else
 * LBP_ERR_WORKSPACE_TOO_SMALL; null pointers give LBP_ERR_INVALID_ARG, an
 * unfilled info LBP_ERR_MISMATCH, a failed copy LBP_ERR_HIP. */
lbp_status lbp_taskmap_to_host(const lbp_plan_info* info, const void* plan_ws_dev, void* host_buf,
                               size_t host_bytes, void* stream);

/* One decode-attention layer (SGLang x HPC-Ops page, "Scheduling around live
 * KV work", second paragraph; vLLM x HPC-Ops page, bullet "Compute and
 * combine"): the persistent attention kernel, then the combine kernel, both
 * on `stream`.  Workgroup b drains bin b: for each descriptor it computes
 * softmax(sm_scale * q k^T) v over the descriptor's tokens for the KV head's
 * whole query group.  A pair with a single descriptor is written to out_dev
 * directly; every descriptor of a pair split over several bins writes its
 * normalised partial output and log-sum-exp to its slot of split_ws_dev, and
 * the combine kernel merges each such pair under the global softmax
 * normalisation into out_dev (BF16, round to nearest even).  A pair with no
 * tokens gets zeros.  k_scale_dev / v_scale_dev are required for FP8 KV and
 * ignored for BF16.  Calls sharing the plan workspace run in stream order
 * (see Concurrency above). */
lbp_status lbp_attend(const lbp_config* cfg, const lbp_plan_info* info,
                      const void* plan_ws_dev, const void* q_dev, const void* k_cache_dev,
                      const void* v_cache_dev, const float* k_scale_dev,
                      const float* v_scale_dev, void* split_ws_dev, size_t split_ws_bytes,
                      void* out_dev, void* stream);

/* lbp_attend as a single launch (DYNAMIC plans; a static plan runs the same
 * two launches as lbp_attend): the workgroup that completes a split pair's
 * last partial merges the pair itself, in split order, through arrival
 * counters kept in the plan workspace (zeroed by the plan, back at zero
 * after every completed launch); a pair of more than 16 partials is merged
 * in two levels (groups of f >= 16 consecutive partials with f * f >= the
 * count, then the group results).  Saves the second launch where pairs are
 * split into few partials; a pair split into many partials puts the chain
 * of the two levels at the end of the kernel, which then costs more than
 * the combine launch.  Launches that share one plan workspace must be
 * ordered on one stream (layers are); concurrent calls need their own plan
 * and split workspaces.  Arguments and results as for lbp_attend (outputs
 * equal up to the rounding of a differently associated merge). */
lbp_status lbp_attend_fused(const lbp_config* cfg, const lbp_plan_info* info,
                            const void* plan_ws_dev, const void* q_dev, const void* k_cache_dev,
                            const void* v_cache_dev, const float* k_scale_dev,
                            const float* v_scale_dev, void* split_ws_dev, size_t split_ws_bytes,
                            void* out_dev, void* stream);

/* The attention kernel and the combine kernel as two launches, for callers
 * that schedule or time them separately (any policy); lbp_combine must
 * follow lbp_attend_partials on the same plan, split workspace and output.
 * lbp_attend_partials runs the persistent attention kernel without the
 * in-kernel merge: a pair whose tokens fit one descriptor is finished in
 * place (its BF16 output is written to out_dev), every descriptor of a pair
 * split over several bins writes its partial to the split buffer, and a
 * pair with no tokens gets zero rows.  lbp_combine merges the split pairs
 * (the plan's split_list) into out_dev.  Split-buffer layout, with
 * C = G * q_len columns per descriptor (column c = query token c / G, head
 * c % G of the KV head's group): o_part[max_desc][C][128] fp32 (normalised
 * partial outputs) at offset 0, then lse_part[max_desc][C] fp32 (base-2
 * log-sum-exp of the sm_scale*log2(e)-scaled scores; -inf for a column with
 * no visible token in the descriptor) at offset align256(max_desc*C*128*4). */
lbp_status lbp_attend_partials(const lbp_config* cfg, const lbp_plan_info* info,
                               const void* plan_ws_dev, const void* q_dev,
                               const void* k_cache_dev, const void* v_cache_dev,
                               const float* k_scale_dev, const float* v_scale_dev,
                               void* split_ws_dev, size_t split_ws_bytes, void* out_dev,
                               void* stream);

/* lbp_attend with an FP8 query, for FP8 KV (cfg->kv_dtype = LBP_KV_FP8_E4M3;
 * otherwise LBP_ERR_UNSUPPORTED).  The SGLang x HPC-Ops page, "A fused
 * attention prologue", has the prologue emit Q in FP8 with a per-token,
 * per-head scale and hand both to the attention kernel without
 * requantization; this entry point takes them in that form:
 *  - q_codes_dev [batch][q_len][num_q_heads][128] uint8 OCP e4m3 codes,
 *  - q_scale_dev [batch][q_len][num_q_heads] fp32; query element =
 *    e4m3(code) * scale.
 * Scores are computed from the K and Q codes on the fp8 MFMA with fp32
 * accumulation, then scaled by q_scale * k_scale * sm_scale; everything else
 * (plan, split buffer, combine, output) is as for lbp_attend.
 * q_scale_dev NULL is LBP_ERR_INVALID_ARG. */
lbp_status lbp_attend_fp8q(const lbp_config* cfg, const lbp_plan_info* info,
                           const void* plan_ws_dev, const uint8_t* q_codes_dev,
                           const float* q_scale_dev, const void* k_cache_dev,
                           const void* v_cache_dev, const float* k_scale_dev,
                           const float* v_scale_dev, void* split_ws_dev, size_t split_ws_bytes,
                           void* out_dev, void* stream);

/* The fused attention prologue of one decode step (SGLang x HPC-Ops page, "A
 * fused attention prologue"; vLLM x HPC-Ops page, the HpcRopeNorm paragraph
 * of the Attention backend section), one launch on `stream`.  For every new
 * token (q_len per request; token j of request r at position
 * p = seq_lens[r] - q_len + j, skipped if p < 0), from its QKV projection:
 *  - query and key heads: RMSNorm over the head's 128 dims
 *    (x / sqrt(mean(x^2) + norm_eps) * weight), then RoPE that rotates each
 *    dim pair (i, i + 64) by the angle of the token's position p (cos/sin
 *    from row min(p, max_position - 1) of rope_cos_sin):
 *    (a, b) -> (a cos - b sin, b cos + a sin);
 *  - the query goes to q_out: BF16 (nearest even), or with q_fp8 = 1 as e4m3
 *    codes with q_scale_out = max|q| / 448 per (request, head) (1 for a zero
 *    row), code = e4m3 nearest to q * 448 / max|q| — the input of
 *    lbp_attend_fp8q;
 *  - the normed, rotated key and the value are written into the paged cache
 *    at page page_table[r][p / 64], slot p % 64, KV head h: BF16 (the value
 *    unchanged), or for an FP8 cache e4m3 codes with k_scale / v_scale =
 *    max|x| / 448 per (token, head).  Positions at or past
 *    64 * cfg->max_pages_per_seq write nothing to the cache.
 * Nothing else in the caches changes.  Host guards: a bad config, batch
 * outside [1, cfg->max_batch], a missing pointer (q_scale_out with q_fp8,
 * k_scale / v_scale with an FP8 cache), max_position < 1, a negative or
 * non-finite norm_eps or a short page-table stride return an error and
 * launch nothing. */
lbp_status lbp_prologue(const lbp_config* cfg, int32_t batch, const lbp_prologue_args* args,
                        void* stream);

/* lbp_attend that also records, for every workgroup b of the attention
 * kernel, four uint64 at trace_dev[4b .. 4b+3]: its start and end on the
 * device's constant-rate real-time clock (s_memrealtime), the hardware-id
 * register in the low and the XCC id in the high 32 bits, and the number of
 * descriptors it drained.  For profiling the balance of the bins (the
 * method's claim that equal bins finish together).  trace_dev must hold
 * 4 * info->num_bins uint64; NULL is LBP_ERR_INVALID_ARG. */
lbp_status lbp_attend_traced(const lbp_config* cfg, const lbp_plan_info* info,
                             const void* plan_ws_dev, const void* q_dev, const void* k_cache_dev,
                             const void* v_cache_dev, const float* k_scale_dev,
                             const float* v_scale_dev, void* split_ws_dev, size_t split_ws_bytes,
                             void* out_dev, uint64_t* trace_dev, void* stream);

/* lbp_attend for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * The same two launches, with the same results bit for bit, but the split
 * buffer lives in a fixed device array of LBP_NOALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on (until the process ends) instead of
 * a caller workspace.  The caller still passes the plan workspace (the input
 * lbp_plan filled), the inputs and the output.  The call allocates nothing:
 * no hipMalloc, hipFree or allocating library routine.  Its first call on a
 * device looks up that device's copy of the array (hipGetSymbolAddress),
 * with the device current.  Nothing in the array needs to start at zero:
 * every partial the combine reads is written by the same call's attention
 * kernel first.  Every call on one GPU shares that GPU's array and leaves the
 * last call's partials in it, so calls that overlap on one GPU (other
 * streams, other threads) race and give wrong results: order them on one
 * stream.  A plan whose split buffer (max_desc x C x 128 x 4 + max_desc x C x
 * 4 bytes, 256-aligned, C = G * q_len; see lbp_query_workspace) exceeds
 * LBP_NOALLOC_SCRATCH_BYTES returns LBP_ERR_SCRATCH_LIMIT and launches
 * nothing.  Other arguments, guards and errors as for lbp_attend. */
lbp_status lbp_attend_noalloc(const lbp_config* cfg, const lbp_plan_info* info,
                              const void* plan_ws_dev, const void* q_dev,
                              const void* k_cache_dev, const void* v_cache_dev,
                              const float* k_scale_dev, const float* v_scale_dev, void* out_dev,
                              void* stream);

lbp_status lbp_combine(const lbp_config* cfg, const lbp_plan_info* info,
                       const void* plan_ws_dev, const void* split_ws_dev,
                       size_t split_ws_bytes, void* out_dev, void* stream);

/* Measurement reference, not part of the attention method: reads `bytes`
 * of device memory at buf_dev once (non-temporal 16-byte loads, workgroup b
 * reading the b-th of `blocks` contiguous chunks) and writes one XOR
 * digest per workgroup to sink_dev[blocks] (int32, caller-owned), so that
 * a timed launch gives this GPU's attainable HBM read rate for streaming
 * traffic like the KV reads of lbp_attend.  buf_dev must be 16-byte aligned
 * and bytes a multiple of 16 (else LBP_ERR_INVALID_ARG); blocks >= 1.
 * Asynchronous on `stream`; LBP_ERR_HIP if the launch is refused. */
lbp_status lbp_read_stream(const void* buf_dev, size_t bytes, int32_t* sink_dev, int32_t blocks,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LBP_H */
