// Host side of liblbp: argument guards, workspace sizing and launches.
// Every entry point checks its arguments before touching the device and
// never synchronises or copies between host and device.
#include <math.h>
#include <string.h>

#include <mutex>

#include "lbp_internal.h"

// The split buffer of lbp_attend_noalloc: one fixed array per GPU, which the
// HIP runtime places in each device's memory when it loads the library's
// code object there.  In host code this name is only a stand-in for the
// symbol: kernels and copies receive the device address that
// hipGetSymbolAddress gives for the current device.
static __device__ __align__(256) unsigned char scratch[LBP_NOALLOC_SCRATCH_BYTES];

namespace lbp {
namespace {

constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices];  // cached per device; 0 = not queried yet

std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxDevices];  // device address of `scratch`; null = not looked up yet

// The current device's copy of `scratch`, looked up once per device (with
// that device current, on its first no-allocation call).
lbp_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return LBP_ERR_HIP;
  if (dev >= kMaxDevices) return LBP_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LBP_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return LBP_OK;
}

lbp_status cu_count(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return LBP_ERR_HIP;
  if (dev < kMaxDevices && g_cu_count[dev] > 0) {
    *out = g_cu_count[dev];
    return LBP_OK;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return LBP_ERR_HIP;
  if (dev < kMaxDevices) g_cu_count[dev] = n;
  *out = n;
  return LBP_OK;
}

lbp_status check_config(const lbp_config* c) {
  if (!c) return LBP_ERR_INVALID_ARG;
  if (c->head_dim != kHeadDim || c->page_size != kPageTokens) return LBP_ERR_UNSUPPORTED;
  if (c->num_q_heads < 1 || c->num_kv_heads < 1) return LBP_ERR_INVALID_ARG;
  if (c->num_q_heads % c->num_kv_heads != 0) return LBP_ERR_INVALID_ARG;
  if (c->num_q_heads / c->num_kv_heads > kMaxGroup) return LBP_ERR_UNSUPPORTED;
  if (c->q_len < 0) return LBP_ERR_INVALID_ARG;
  if (int64_t(c->num_q_heads / c->num_kv_heads) * (c->q_len > 1 ? c->q_len : 1) >
      LBP_MAX_QUERY_COLUMNS)
    return LBP_ERR_UNSUPPORTED;
  if (c->max_batch < 1 || c->max_pages_per_seq < 1) return LBP_ERR_INVALID_ARG;
  if (c->num_workgroups < 0 || c->min_tiles_per_bin < 0) return LBP_ERR_INVALID_ARG;
  if (c->kv_dtype != LBP_KV_BF16 && c->kv_dtype != LBP_KV_FP8_E4M3) return LBP_ERR_UNSUPPORTED;
  if (!(c->sm_scale > 0.f) || !isfinite(c->sm_scale)) return LBP_ERR_INVALID_ARG;
  // all tile, token and descriptor counts must fit in int32
  const int64_t pairs = int64_t(c->num_kv_heads) * c->max_batch;
  if (int64_t(c->max_pages_per_seq) * kPageTokens > INT32_MAX / 2) return LBP_ERR_UNSUPPORTED;
  if (pairs * c->max_pages_per_seq > INT32_MAX / 2) return LBP_ERR_UNSUPPORTED;
  if (c->num_workgroups > (1 << 20)) return LBP_ERR_UNSUPPORTED;
  return LBP_OK;
}

// Query tokens per request and query columns per KV head.
int q_len_of(const lbp_config* c) { return c->q_len > 1 ? c->q_len : 1; }
int ncols_of(const lbp_config* c) { return c->num_q_heads / c->num_kv_heads * q_len_of(c); }

lbp_status resolve_bins(const lbp_config* c, int* W) {
  if (c->num_workgroups > 0) {
    *W = c->num_workgroups;
    return LBP_OK;
  }
  return cu_count(W);
}

// Grid and descriptor capacity of a (policy, param) at a given batch.
lbp_status plan_shape(const lbp_config* c, int policy, int param, int batch, int* num_bins,
                      int* max_desc, int* splits_per_pair, int* used_param) {
  const int64_t pairs = int64_t(c->num_kv_heads) * batch;
  if (policy == LBP_POLICY_DYNAMIC) {
    int W;
    lbp_status st = resolve_bins(c, &W);
    if (st != LBP_OK) return st;
    int F = param > 0 ? param : (c->min_tiles_per_bin > 0 ? c->min_tiles_per_bin : kDefaultMinTiles);
    if (param < 0) return LBP_ERR_INVALID_ARG;
    *num_bins = W;
    *max_desc = int(pairs + W - 1);   // a boundary between bins adds at most one descriptor
    *splits_per_pair = 0;
    *used_param = F;
    return LBP_OK;
  }
  if (param < 1) return LBP_ERR_INVALID_ARG;
  int S;
  if (policy == LBP_POLICY_STATIC_SPLITS) {
    if (param > 4096) return LBP_ERR_UNSUPPORTED;
    S = param;
  } else if (policy == LBP_POLICY_STATIC_CHUNK) {
    S = (c->max_pages_per_seq + param - 1) / param;
  } else {
    return LBP_ERR_INVALID_ARG;
  }
  if (pairs * S > INT32_MAX / 4) return LBP_ERR_UNSUPPORTED;
  *num_bins = int(pairs * S);
  *max_desc = int(pairs * S);
  *splits_per_pair = S;
  *used_param = param;
  return LBP_OK;
}

lbp_status check_info(const lbp_config* c, const lbp_plan_info* info) {
  if (!info || info->magic != LBP_PLAN_MAGIC) return LBP_ERR_MISMATCH;
  if (info->num_kv_heads != c->num_kv_heads || info->num_q_heads != c->num_q_heads)
    return LBP_ERR_MISMATCH;
  if (info->batch < 1 || info->batch > c->max_batch) return LBP_ERR_MISMATCH;
  if (info->num_bins < 1 || info->max_desc < 0 || !info->page_table_dev) return LBP_ERR_MISMATCH;
  return LBP_OK;
}

lbp_status build_plan(const lbp_config* cfg, int policy, int param, const int32_t* seq_lens,
                      int32_t batch, const int32_t* page_table, int64_t stride, void* ws,
                      size_t ws_bytes, lbp_plan_info* info, void* stream) {
  lbp_status st = check_config(cfg);
  if (st != LBP_OK) return st;
  if (!seq_lens || !page_table || !ws || !info) return LBP_ERR_INVALID_ARG;
  if (batch < 1 || batch > cfg->max_batch) return LBP_ERR_INVALID_ARG;
  if (stride < cfg->max_pages_per_seq) return LBP_ERR_INVALID_ARG;
  int num_bins, max_desc, spp, used;
  st = plan_shape(cfg, policy, param, batch, &num_bins, &max_desc, &spp, &used);
  if (st != LBP_OK) return st;
  const int npairs = cfg->num_kv_heads * batch;
  const lbp_plan_offsets off = plan_layout(policy, num_bins, max_desc, npairs);
  if (ws_bytes < off.total) return LBP_ERR_WORKSPACE_TOO_SMALL;

  char* base = static_cast<char*>(ws);
  PlanArgs a;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.num_kv_heads = cfg->num_kv_heads;
  a.num_bins = num_bins;
  a.policy = policy;
  a.param = used;
  a.splits_per_pair = spp;
  a.max_tokens = cfg->max_pages_per_seq * kPageTokens;
  a.header = reinterpret_cast<int32_t*>(base + off.header);
  a.bin_offset = reinterpret_cast<int32_t*>(base + off.bin_offset);
  a.bin_first = reinterpret_cast<int32_t*>(base + off.bin_first);
  a.page_table = page_table;
  a.page_table_stride = stride;
  a.desc = reinterpret_cast<int32_t*>(base + off.desc);
  a.pair_first = reinterpret_cast<int32_t*>(base + off.pair_first);
  a.pair_count = reinterpret_cast<int32_t*>(base + off.pair_count);
  a.scratch = reinterpret_cast<int32_t*>(base + off.scratch);
  a.split_list = reinterpret_cast<int32_t*>(base + off.split_list);
  a.max_split = max_split_pairs(policy, num_bins, npairs);
  a.arrive = reinterpret_cast<int32_t*>(base + off.arrive);
  a.arrive_words = arrive_words(policy, max_desc);
  if (launch_plan(a, static_cast<hipStream_t>(stream)) != hipSuccess) return LBP_ERR_HIP;

  lbp_plan_info out;
  memset(&out, 0, sizeof(out));
  out.magic = LBP_PLAN_MAGIC;
  out.policy = policy;
  out.param = used;
  out.batch = batch;
  out.num_kv_heads = cfg->num_kv_heads;
  out.num_q_heads = cfg->num_q_heads;
  out.num_bins = num_bins;
  out.max_desc = max_desc;
  out.plan_bytes = off.total;
  out.page_table_dev = page_table;
  out.page_table_stride = stride;
  *info = out;
  return LBP_OK;
}

lbp_plan_offsets offsets_of(const lbp_plan_info* info) {
  return plan_layout(info->policy, info->num_bins, info->max_desc, info->num_kv_heads * info->batch);
}

lbp_status check_split(const lbp_config* cfg, const lbp_plan_info* info, size_t bytes) {
  return bytes < split_bytes(info->max_desc, ncols_of(cfg)) ? LBP_ERR_WORKSPACE_TOO_SMALL : LBP_OK;
}

}  // namespace
}  // namespace lbp

using namespace lbp;

extern "C" {

const char* lbp_status_string(lbp_status s) {
  switch (s) {
    case LBP_OK: return "LBP_OK";
    case LBP_ERR_INVALID_ARG: return "LBP_ERR_INVALID_ARG";
    case LBP_ERR_UNSUPPORTED: return "LBP_ERR_UNSUPPORTED";
    case LBP_ERR_WORKSPACE_TOO_SMALL: return "LBP_ERR_WORKSPACE_TOO_SMALL";
    case LBP_ERR_MISMATCH: return "LBP_ERR_MISMATCH";
    case LBP_ERR_HIP: return "LBP_ERR_HIP";
    case LBP_ERR_SCRATCH_LIMIT: return "LBP_ERR_SCRATCH_LIMIT";
  }
  return "LBP_ERR_UNKNOWN";
}

int32_t lbp_version(void) { return LBP_VERSION; }

lbp_status lbp_query_workspace(const lbp_config* cfg, int32_t policy, int32_t param,
                               size_t* plan_bytes, size_t* split_ws) {
  lbp_status st = check_config(cfg);
  if (st != LBP_OK) return st;
  if (!plan_bytes || !split_ws) return LBP_ERR_INVALID_ARG;
  int num_bins, max_desc, spp, used;
  st = plan_shape(cfg, policy, param, cfg->max_batch, &num_bins, &max_desc, &spp, &used);
  if (st != LBP_OK) return st;
  *plan_bytes = plan_layout(policy, num_bins, max_desc, cfg->num_kv_heads * cfg->max_batch).total;
  *split_ws = split_bytes(max_desc, ncols_of(cfg));
  return LBP_OK;
}

lbp_status lbp_plan(const lbp_config* cfg, const int32_t* seq_lens_dev, int32_t batch,
                    const int32_t* page_table_dev, int64_t page_table_stride, void* plan_ws_dev,
                    size_t plan_ws_bytes, lbp_plan_info* info, void* stream) {
  const int F = cfg && cfg->min_tiles_per_bin > 0 ? cfg->min_tiles_per_bin : kDefaultMinTiles;
  return build_plan(cfg, LBP_POLICY_DYNAMIC, F, seq_lens_dev, batch, page_table_dev,
                    page_table_stride, plan_ws_dev, plan_ws_bytes, info, stream);
}

lbp_status lbp_plan_static(const lbp_config* cfg, int32_t policy, int32_t param,
                           const int32_t* seq_lens_dev, int32_t batch,
                           const int32_t* page_table_dev, int64_t page_table_stride,
                           void* plan_ws_dev, size_t plan_ws_bytes, lbp_plan_info* info,
                           void* stream) {
  if (policy != LBP_POLICY_STATIC_SPLITS && policy != LBP_POLICY_STATIC_CHUNK)
    return LBP_ERR_INVALID_ARG;
  return build_plan(cfg, policy, param, seq_lens_dev, batch, page_table_dev, page_table_stride,
                    plan_ws_dev, plan_ws_bytes, info, stream);
}

lbp_status lbp_plan_layout(const lbp_plan_info* info, lbp_plan_offsets* offsets) {
  if (!info || !offsets) return LBP_ERR_INVALID_ARG;
  if (info->magic != LBP_PLAN_MAGIC) return LBP_ERR_MISMATCH;
  *offsets = offsets_of(info);
  return LBP_OK;
}

lbp_status lbp_taskmap_to_host(const lbp_plan_info* info, const void* plan_ws_dev, void* host_buf,
                               size_t host_bytes, void* stream) {
  if (!info || !plan_ws_dev || !host_buf) return LBP_ERR_INVALID_ARG;
  if (info->magic != LBP_PLAN_MAGIC) return LBP_ERR_MISMATCH;
  const uint64_t total = offsets_of(info).total;
  if (host_bytes < total) return LBP_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(host_buf, plan_ws_dev, total, hipMemcpyDeviceToHost, s) != hipSuccess)
    return LBP_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return LBP_ERR_HIP;
  return LBP_OK;
}

// The attention kernel alone (fuse = false) or, for a dynamic plan with
// fuse = true, the attention kernel that also merges the split pairs.
static lbp_status attend_impl(const lbp_config* cfg, const lbp_plan_info* info,
                              const void* plan_ws_dev, const void* q_dev, const void* k_cache_dev,
                              const void* v_cache_dev, const float* k_scale_dev,
                              const float* v_scale_dev, void* split_ws_dev, size_t split_ws_bytes,
                              void* out_dev, uint64_t* trace_dev, bool fuse, void* stream,
                              const float* q_scale_dev = nullptr) {
  lbp_status st = check_config(cfg);
  if (st != LBP_OK) return st;
  if ((st = check_info(cfg, info)) != LBP_OK) return st;
  if (!plan_ws_dev || !q_dev || !k_cache_dev || !v_cache_dev || !split_ws_dev || !out_dev)
    return LBP_ERR_INVALID_ARG;
  if (cfg->kv_dtype == LBP_KV_FP8_E4M3 && (!k_scale_dev || !v_scale_dev))
    return LBP_ERR_INVALID_ARG;
  if ((st = check_split(cfg, info, split_ws_bytes)) != LBP_OK) return st;

  const lbp_plan_offsets off = offsets_of(info);
  const char* pb = static_cast<const char*>(plan_ws_dev);
  const int G = cfg->num_q_heads / cfg->num_kv_heads;
  AttendArgs a;
  a.bin_offset = reinterpret_cast<const int32_t*>(pb + off.bin_offset);
  a.bin_first = reinterpret_cast<const int32_t*>(pb + off.bin_first);
  a.desc = reinterpret_cast<const int32_t*>(pb + off.desc);
  a.pair_count = reinterpret_cast<const int32_t*>(pb + off.pair_count);
  a.pair_first = reinterpret_cast<const int32_t*>(pb + off.pair_first);
  a.page_table = info->page_table_dev;
  a.page_table_stride = info->page_table_stride;
  a.q = q_dev;
  a.q_scale = q_scale_dev;
  a.k_cache = k_cache_dev;
  a.v_cache = v_cache_dev;
  a.k_scale = cfg->kv_dtype == LBP_KV_FP8_E4M3 ? k_scale_dev : nullptr;
  a.v_scale = cfg->kv_dtype == LBP_KV_FP8_E4M3 ? v_scale_dev : nullptr;
  a.o_part = static_cast<float*>(split_ws_dev);
  a.lse_part = reinterpret_cast<float*>(static_cast<char*>(split_ws_dev) +
                                        split_lse_offset(info->max_desc, ncols_of(cfg)));
  // buffer resources address the split buffer with 32-bit offsets
  const uint64_t o_bytes = split_lse_offset(info->max_desc, ncols_of(cfg));
  const uint64_t lse_bytes = uint64_t(info->max_desc) * ncols_of(cfg) * 4;
  if (fuse && info->policy == LBP_POLICY_DYNAMIC && o_bytes > uint64_t(INT32_MAX))
    return LBP_ERR_UNSUPPORTED;
  a.o_part_bytes = int32_t(o_bytes < uint64_t(INT32_MAX) ? o_bytes : uint64_t(INT32_MAX));
  a.lse_part_bytes = int32_t(lse_bytes < uint64_t(INT32_MAX) ? lse_bytes : uint64_t(INT32_MAX));
  a.out = out_dev;
  a.trace = trace_dev;
  a.num_bins = info->num_bins;
  // Dynamic plans with more bins than CUs run one persistent workgroup per
  // CU that takes bins in order from the ticket counter; otherwise (and for
  // the static comparison plans, which are ordinary grids) one workgroup
  // per bin.
  int grid = info->num_bins;
  a.grab_counter = nullptr;
  if (info->policy == LBP_POLICY_DYNAMIC) {
    int cus = 0;
    if ((st = cu_count(&cus)) != LBP_OK) return st;
    if (info->num_bins > cus) {
      grid = cus;
      a.grab_counter = reinterpret_cast<int32_t*>(const_cast<char*>(pb) + off.header) + kHdrTicket;
    }
  }
  a.fuse = fuse && info->policy == LBP_POLICY_DYNAMIC;
  int32_t* arrive = reinterpret_cast<int32_t*>(const_cast<char*>(pb) + off.arrive);
  a.arrive_pair = a.fuse ? arrive : nullptr;
  a.arrive_group = a.fuse ? arrive + info->max_desc : nullptr;
  a.batch = info->batch;
  a.num_q_heads = cfg->num_q_heads;
  a.num_kv_heads = cfg->num_kv_heads;
  a.group = G;
  a.q_len = q_len_of(cfg);
  a.ncols = ncols_of(cfg);
  a.scale_log2 = cfg->sm_scale * 1.4426950408889634f;
  const AttendKind kind = q_scale_dev ? kAttendFp8Q8
                          : cfg->kv_dtype == LBP_KV_FP8_E4M3 ? kAttendFp8 : kAttendBf16;
  if (launch_attend(a, kind, grid, static_cast<hipStream_t>(stream)) != hipSuccess)
    return LBP_ERR_HIP;
  return LBP_OK;
}

lbp_status lbp_attend_partials(const lbp_config* cfg, const lbp_plan_info* info,
                               const void* plan_ws_dev, const void* q_dev,
                               const void* k_cache_dev, const void* v_cache_dev,
                               const float* k_scale_dev, const float* v_scale_dev,
                               void* split_ws_dev, size_t split_ws_bytes, void* out_dev,
                               void* stream) {
  return attend_impl(cfg, info, plan_ws_dev, q_dev, k_cache_dev, v_cache_dev, k_scale_dev,
                     v_scale_dev, split_ws_dev, split_ws_bytes, out_dev, nullptr, false, stream);
}

lbp_status lbp_combine(const lbp_config* cfg, const lbp_plan_info* info, const void* plan_ws_dev,
                       const void* split_ws_dev, size_t split_ws_bytes, void* out_dev,
                       void* stream) {
  lbp_status st = check_config(cfg);
  if (st != LBP_OK) return st;
  if ((st = check_info(cfg, info)) != LBP_OK) return st;
  if (!plan_ws_dev || !split_ws_dev || !out_dev) return LBP_ERR_INVALID_ARG;
  if ((st = check_split(cfg, info, split_ws_bytes)) != LBP_OK) return st;
  const lbp_plan_offsets off = offsets_of(info);
  const char* pb = static_cast<const char*>(plan_ws_dev);
  const int G = cfg->num_q_heads / cfg->num_kv_heads;
  CombineArgs a;
  a.header = reinterpret_cast<const int32_t*>(pb + off.header);
  a.split_list = reinterpret_cast<const int32_t*>(pb + off.split_list);
  a.o_part = static_cast<const float*>(split_ws_dev);
  a.lse_part = reinterpret_cast<const float*>(static_cast<const char*>(split_ws_dev) +
                                              split_lse_offset(info->max_desc, ncols_of(cfg)));
  a.out = out_dev;
  a.batch = info->batch;
  a.num_q_heads = cfg->num_q_heads;
  a.num_kv_heads = cfg->num_kv_heads;
  a.group = G;
  a.q_len = q_len_of(cfg);
  a.ncols = ncols_of(cfg);
  const int max_split =
      max_split_pairs(info->policy, info->num_bins, cfg->num_kv_heads * info->batch);
  if (launch_combine(a, max_split, static_cast<hipStream_t>(stream)) != hipSuccess)
    return LBP_ERR_HIP;
  return LBP_OK;
}

// The attention kernel, then (unless it merged the split pairs itself, which
// only the fused entry point on a dynamic plan asks for) the combine kernel.
static lbp_status attend_full(const lbp_config* cfg, const lbp_plan_info* info,
                              const void* plan_ws_dev, const void* q_dev, const void* k_cache_dev,
                              const void* v_cache_dev, const float* k_scale_dev,
                              const float* v_scale_dev, void* split_ws_dev, size_t split_ws_bytes,
                              void* out_dev, uint64_t* trace_dev, bool fuse, void* stream) {
  if (!info) return LBP_ERR_MISMATCH;
  lbp_status st = attend_impl(cfg, info, plan_ws_dev, q_dev, k_cache_dev, v_cache_dev,
                              k_scale_dev, v_scale_dev, split_ws_dev, split_ws_bytes, out_dev,
                              trace_dev, fuse, stream);
  if (st != LBP_OK || (fuse && info->policy == LBP_POLICY_DYNAMIC)) return st;
  return lbp_combine(cfg, info, plan_ws_dev, split_ws_dev, split_ws_bytes, out_dev, stream);
}

lbp_status lbp_attend(const lbp_config* cfg, const lbp_plan_info* info, const void* plan_ws_dev,
                      const void* q_dev, const void* k_cache_dev, const void* v_cache_dev,
                      const float* k_scale_dev, const float* v_scale_dev, void* split_ws_dev,
                      size_t split_ws_bytes, void* out_dev, void* stream) {
  return attend_full(cfg, info, plan_ws_dev, q_dev, k_cache_dev, v_cache_dev, k_scale_dev,
                     v_scale_dev, split_ws_dev, split_ws_bytes, out_dev, nullptr, false, stream);
}

lbp_status lbp_attend_noalloc(const lbp_config* cfg, const lbp_plan_info* info,
                              const void* plan_ws_dev, const void* q_dev,
                              const void* k_cache_dev, const void* v_cache_dev,
                              const float* k_scale_dev, const float* v_scale_dev, void* out_dev,
                              void* stream) {
  // every guard of lbp_attend that needs no device comes first, then the
  // size of the split buffer against the fixed array, then its address
  lbp_status st = check_config(cfg);
  if (st != LBP_OK) return st;
  if ((st = check_info(cfg, info)) != LBP_OK) return st;
  if (!plan_ws_dev || !q_dev || !k_cache_dev || !v_cache_dev || !out_dev)
    return LBP_ERR_INVALID_ARG;
  if (cfg->kv_dtype == LBP_KV_FP8_E4M3 && (!k_scale_dev || !v_scale_dev))
    return LBP_ERR_INVALID_ARG;
  if (split_bytes(info->max_desc, ncols_of(cfg)) > LBP_NOALLOC_SCRATCH_BYTES)
    return LBP_ERR_SCRATCH_LIMIT;
  void* split = nullptr;
  if ((st = scratch_address(&split)) != LBP_OK) return st;
  return attend_full(cfg, info, plan_ws_dev, q_dev, k_cache_dev, v_cache_dev, k_scale_dev,
                     v_scale_dev, split, LBP_NOALLOC_SCRATCH_BYTES, out_dev, nullptr, false,
                     stream);
}

lbp_status lbp_attend_fused(const lbp_config* cfg, const lbp_plan_info* info,
                            const void* plan_ws_dev, const void* q_dev, const void* k_cache_dev,
                            const void* v_cache_dev, const float* k_scale_dev,
                            const float* v_scale_dev, void* split_ws_dev, size_t split_ws_bytes,
                            void* out_dev, void* stream) {
  return attend_full(cfg, info, plan_ws_dev, q_dev, k_cache_dev, v_cache_dev, k_scale_dev,
                     v_scale_dev, split_ws_dev, split_ws_bytes, out_dev, nullptr, true, stream);
}

lbp_status lbp_attend_traced(const lbp_config* cfg, const lbp_plan_info* info,
                             const void* plan_ws_dev, const void* q_dev, const void* k_cache_dev,
                             const void* v_cache_dev, const float* k_scale_dev,
                             const float* v_scale_dev, void* split_ws_dev, size_t split_ws_bytes,
                             void* out_dev, uint64_t* trace_dev, void* stream) {
  if (!trace_dev) return LBP_ERR_INVALID_ARG;
  return attend_full(cfg, info, plan_ws_dev, q_dev, k_cache_dev, v_cache_dev, k_scale_dev,
                     v_scale_dev, split_ws_dev, split_ws_bytes, out_dev, trace_dev, false, stream);
}

lbp_status lbp_attend_fp8q(const lbp_config* cfg, const lbp_plan_info* info,
                           const void* plan_ws_dev, const uint8_t* q_codes_dev,
                           const float* q_scale_dev, const void* k_cache_dev,
                           const void* v_cache_dev, const float* k_scale_dev,
                           const float* v_scale_dev, void* split_ws_dev, size_t split_ws_bytes,
                           void* out_dev, void* stream) {
  if (!cfg) return LBP_ERR_INVALID_ARG;
  if (cfg->kv_dtype != LBP_KV_FP8_E4M3) return LBP_ERR_UNSUPPORTED;
  if (!q_scale_dev || !info) return LBP_ERR_INVALID_ARG;
  lbp_status st = attend_impl(cfg, info, plan_ws_dev, q_codes_dev, k_cache_dev, v_cache_dev,
                              k_scale_dev, v_scale_dev, split_ws_dev, split_ws_bytes, out_dev,
                              nullptr, false, stream, q_scale_dev);
  if (st != LBP_OK) return st;
  return lbp_combine(cfg, info, plan_ws_dev, split_ws_dev, split_ws_bytes, out_dev, stream);
}

lbp_status lbp_prologue(const lbp_config* cfg, int32_t batch, const lbp_prologue_args* args,
                        void* stream) {
  lbp_status st = check_config(cfg);
  if (st != LBP_OK) return st;
  if (!args || batch < 1 || batch > cfg->max_batch) return LBP_ERR_INVALID_ARG;
  const lbp_prologue_args& p = *args;
  const bool kv_fp8 = cfg->kv_dtype == LBP_KV_FP8_E4M3;
  if (!p.qkv || !p.seq_lens || !p.page_table || !p.q_norm_weight || !p.k_norm_weight ||
      !p.rope_cos_sin || !p.q_out || !p.k_cache || !p.v_cache)
    return LBP_ERR_INVALID_ARG;
  if (p.q_fp8 != 0 && p.q_fp8 != 1) return LBP_ERR_INVALID_ARG;
  if (p.q_fp8 && !p.q_scale_out) return LBP_ERR_INVALID_ARG;
  if (kv_fp8 && (!p.k_scale || !p.v_scale)) return LBP_ERR_INVALID_ARG;
  if (p.max_position < 1 || !(p.norm_eps >= 0.f) || !isfinite(p.norm_eps))
    return LBP_ERR_INVALID_ARG;
  if (p.page_table_stride < cfg->max_pages_per_seq) return LBP_ERR_INVALID_ARG;
  PrologueArgs a;
  a.qkv = p.qkv;
  a.seq_lens = p.seq_lens;
  a.page_table = p.page_table;
  a.page_table_stride = p.page_table_stride;
  a.q_norm_weight = p.q_norm_weight;
  a.k_norm_weight = p.k_norm_weight;
  a.rope_cos_sin = p.rope_cos_sin;
  a.max_position = p.max_position;
  a.norm_eps = p.norm_eps;
  a.q_fp8 = p.q_fp8;
  a.kv_fp8 = kv_fp8;
  a.q_out = p.q_out;
  a.q_scale_out = p.q_scale_out;
  a.k_cache = p.k_cache;
  a.v_cache = p.v_cache;
  a.k_scale = kv_fp8 ? p.k_scale : nullptr;
  a.v_scale = kv_fp8 ? p.v_scale : nullptr;
  a.batch = batch;
  a.num_q_heads = cfg->num_q_heads;
  a.num_kv_heads = cfg->num_kv_heads;
  a.q_len = q_len_of(cfg);
  a.max_tokens = cfg->max_pages_per_seq * kPageTokens;
  if (launch_prologue(a, static_cast<hipStream_t>(stream)) != hipSuccess) return LBP_ERR_HIP;
  return LBP_OK;
}

lbp_status lbp_read_stream(const void* buf_dev, size_t bytes, int32_t* sink_dev, int32_t blocks,
                           void* stream) {
  if (!buf_dev || !sink_dev || blocks < 1 || bytes % 16 != 0) return LBP_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(buf_dev) % 16 != 0) return LBP_ERR_INVALID_ARG;
  if (launch_read_stream(buf_dev, int64_t(bytes / 16), sink_dev, blocks,
                         static_cast<hipStream_t>(stream)) != hipSuccess)
    return LBP_ERR_HIP;
  return LBP_OK;
}

}  // extern "C"
