// C ABI of libpa: argument validation, the pool descriptor, dispatch to the
// HIP kernels, device status and kernel timing.  Nothing throws across the ABI.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/pa.h"
#include "block_manager.hpp"
#include "kernels.hpp"

namespace {

// A fixed buffer, so that reporting a failure allocates nothing.
thread_local char g_last_error[512];

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

constexpr int kMinSplitTokens = 1024;  // shorter contexts always run in one pass

}  // namespace

// Split-context partials of pa_decode_noalloc: a fixed device array, one copy
// per GPU, held until the process ends.  Host code never uses its name as an
// address (on the host it is only a stand-in): the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) uint8_t scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
hipError_t g_scratch_err[kMaxDevices] = {};

// Looks up (once per device) the device address of `scratch` on device `dev`,
// which must be current.  Returns null if the lookup failed.
void* scratch_on_current_device(int dev, hipError_t* err) {
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev] && g_scratch_err[dev] == hipSuccess) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e == hipSuccess && ptr) g_scratch_ptr[dev] = ptr;
    else g_scratch_err[dev] = e != hipSuccess ? e : hipErrorInvalidSymbol;
  }
  *err = g_scratch_err[dev];
  return g_scratch_ptr[dev];
}

}  // namespace

static_assert(PA_DTYPE_FP16 == pa::kF16 && PA_DTYPE_FP8_E4M3 == pa::kF8 && PA_DTYPE_INT8 == pa::kI8,
              "dtype codes are the kernels' element kinds");

struct pa_pool {
  int32_t layers, kv_heads, head_dim, block_size, dtype, num_blocks, elem_bytes;
  uint64_t tile_bytes, kv_bytes, scales_offset, status_offset, total_bytes;
  pa::BlockManager bm;
  bool bound = false;
  int device = -1;
  int num_cus = 256;
  int32_t load_policy = PA_LOADS_AUTO;  // K/V loads of the decode kernel
  void* scratch = nullptr;           // device address of `scratch` on `device`
  hipError_t scratch_err = hipSuccess;
  pa::PoolGeom geom{};
  // kernel timing
  bool profiling = false;
  int32_t max_records = 0;
  int32_t every = 1;      // time one launch in `every`
  int64_t launches = 0;   // launches seen since pa_profile_begin
  std::vector<hipEvent_t> ev;  // 4 per record: decode start/end, reduce start/end (if any)
  std::vector<int8_t> has_reduce;
  int32_t n_records = 0;
  // multi-token work items: a ring of pinned host staging buffers, each
  // reused once the event of the upload that last read it has completed (so
  // the host can run several launches ahead of the device)
  struct Staging {
    int32_t* host = nullptr;
    size_t cap = 0;  // int32 entries
    hipEvent_t done = nullptr;
  };
  static constexpr int kStagingRing = 16;
  Staging mt_ring[kStagingRing];
  int mt_next = 0;

  pa_pool(int32_t L, int32_t H, int32_t D, int32_t B, int32_t dt, int32_t N)
      : layers(L), kv_heads(H), head_dim(D), block_size(B), dtype(dt), num_blocks(N),
        elem_bytes(dt == PA_DTYPE_FP16 ? 2 : 1), bm(N, B) {
    tile_bytes = static_cast<uint64_t>(B) * D * elem_bytes;
    kv_bytes = 2ull * L * N * H * tile_bytes;
    scales_offset = align_up(kv_bytes, 256);
    status_offset = align_up(scales_offset + 24ull * L * H, 256);  // six fp32 per (layer, head)
    total_bytes = status_offset + 256;
  }
  ~pa_pool() {
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
    for (Staging& st : mt_ring) {
      if (st.done) {
        (void)hipEventSynchronize(st.done);
        (void)hipEventDestroy(st.done);
      }
      if (st.host) (void)hipHostFree(st.host);
    }
  }
};

namespace {

// Launch shape of one decode: single pass (C = 1) or chunks of P tokens.
struct Plan {
  bool partial;
  int mode;  // pa::DecodeLaunch::mode
  int partition_tokens;
  int num_partitions;
  int chunks_per_wave;
  int waves_per_unit;
  uint64_t ws_bytes, off_l, off_o;
};

constexpr int kModeSingle = 0, kModeSplit4 = 1, kModeSplit1 = 2, kModePrivate = 3;

int make_plan(const pa_pool* p, int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks,
              int32_t partition_tokens, Plan* out) {
  if (max_blocks < 1 || static_cast<int64_t>(max_blocks) * p->block_size > 0x7FFFFFFF)
    return fail(PA_ERR_INVALID, "max_blocks %d out of range", max_blocks);
  if (num_seqs < 0) return fail(PA_ERR_INVALID, "num_seqs %d < 0", num_seqs);
  if (num_q_heads < 1 || num_q_heads % p->kv_heads != 0)
    return fail(PA_ERR_INVALID, "num_q_heads %d is not a multiple of kv_heads %d", num_q_heads,
                p->kv_heads);
  const int group = num_q_heads / p->kv_heads;
  if (group > 32) return fail(PA_ERR_INVALID, "query heads per KV head %d > 32", group);
  const int64_t t_cap = static_cast<int64_t>(max_blocks) * p->block_size;
  const int64_t units = static_cast<int64_t>(num_seqs) * p->kv_heads;
  int P;
  if (partition_tokens == -1) {
    P = 0;
  } else if (partition_tokens == 0) {
    // One workgroup per (sequence, KV head) streams its whole context at full
    // rate once every CU has one; with fewer units, split each context into
    // just enough chunks to give every CU a workgroup (measured on MI355X:
    // more, shorter chunks only add partial writes and start-up latency).
    // Wide head groups (more than 16 query heads per KV head) do twice the
    // math per byte and want two workgroups per CU.
    P = 0;
    const int64_t target = static_cast<int64_t>(p->num_cus) * (group > 16 ? 2 : 1);
    if (t_cap > kMinSplitTokens && units < target) {
      const int64_t parts = (target + units - 1) / units;
      const int64_t len = (t_cap + parts - 1) / parts;
      const int64_t chunk = align_up(static_cast<uint64_t>(len), 64);  // four waves x 16 tokens
      if (chunk < t_cap) P = static_cast<int>(chunk);
    }
  } else {
    if (partition_tokens % 16 != 0 || partition_tokens % p->block_size != 0)
      return fail(PA_ERR_INVALID, "partition_tokens %d must be a multiple of 16 and of block_size %d",
                  partition_tokens, p->block_size);
    P = partition_tokens;
  }
  Plan pl{};
  if (P == 0) {
    pl.partial = false;
    pl.mode = kModeSingle;
    pl.partition_tokens = static_cast<int>(align_up(static_cast<uint64_t>(t_cap), 16));
    pl.num_partitions = 1;
    pl.chunks_per_wave = 1;
    pl.waves_per_unit = 1;
  } else {
    pl.partial = true;
    pl.partition_tokens = P;
    const int64_t C = (t_cap + P - 1) / P;
    pl.num_partitions = static_cast<int>(C);
    // Schedule: about eight waves per CU.  With at least one chunk per wave
    // available, each wave streams a run of k whole chunks on its own (no
    // merges); otherwise the four waves of a workgroup share every chunk of a
    // run and merge at each chunk end (needs P to be a multiple of 64).
    const int64_t target_waves = static_cast<int64_t>(p->num_cus) * 8;
    const int64_t chunks = units * C;
    int64_t k;
    if (chunks >= target_waves || P % 64 != 0) {
      pl.mode = kModeSplit1;
      k = chunks / target_waves;
    } else {
      pl.mode = kModeSplit4;
      k = 4 * chunks / target_waves;
    }
    k = k < 1 ? 1 : (k > C ? C : k);
    pl.chunks_per_wave = static_cast<int>(k);
    pl.waves_per_unit = static_cast<int>((C + k - 1) / k);
    // A remainder of at most k/4 chunks joins the unit's last run instead of
    // forming a run of its own: that run would add a second, nearly empty
    // round of workgroups when the runs exactly fill the device (for example
    // 257 chunks of 512 tokens in runs of 8).
    const int64_t rem = C % k;
    if (C > k && rem != 0 && rem * 4 <= k) pl.waves_per_unit = static_cast<int>(C / k);
    const uint64_t rows = static_cast<uint64_t>(num_seqs) * num_q_heads * pl.num_partitions;
    pl.off_l = align_up(rows * 4, 256);
    pl.off_o = pl.off_l + align_up(rows * 4, 256);
    pl.ws_bytes = pl.off_o + align_up(rows * p->head_dim * 4, 256);
  }
  *out = pl;
  return PA_OK;
}

int check_bound(const pa_pool* p) {
  if (!p) return fail(PA_ERR_INVALID, "pool is NULL");
  if (!p->bound) return fail(PA_ERR_UNBOUND, "pool has no device memory (call pa_pool_bind)");
  return PA_OK;
}

int check_layer(const pa_pool* p, int32_t layer) {
  if (layer < 0 || layer >= p->layers)
    return fail(PA_ERR_INVALID, "layer %d outside [0, %d)", layer, p->layers);
  return PA_OK;
}

int bm_status(pa::BmStatus s, int32_t seq) {
  switch (s) {
    case pa::BmStatus::kOk: return PA_OK;
    case pa::BmStatus::kNoBlocks: return fail(PA_ERR_NO_BLOCKS, "not enough free blocks for sequence %d", seq);
    case pa::BmStatus::kBadSeq: return fail(PA_ERR_BAD_SEQ, "unknown or freed sequence %d", seq);
    default: return fail(PA_ERR_INVALID, "invalid argument for sequence %d", seq);
  }
}

// Whether decode launches use ordinary (cached) K/V loads: forced by the
// pool's policy, or, by default, when the pool's used blocks have on average
// at least 1.5 holders (sequences whose tables name them), i.e. when a
// launch's sequences are likely to read many blocks more than once.
bool use_cached_loads(const pa_pool* p) {
  if (p->load_policy == PA_LOADS_STREAMING) return false;
  if (p->load_policy == PA_LOADS_CACHED) return true;
  const int64_t used = p->num_blocks - p->bm.free_count();
  return used > 0 && 2 * p->bm.table_entries() >= 3 * used;
}

pa::DecodeLaunch make_launch(int32_t layer, const void* q, int32_t num_q_heads,
                             const int32_t* tables, int32_t max_blocks, const int32_t* lens,
                             int32_t num_seqs, const int32_t* order, float scale, const Plan& pl,
                             void* out, void* workspace) {
  pa::DecodeLaunch d{};
  d.layer = layer;
  d.q = q;
  d.tables = tables;
  d.lens = lens;
  d.order = order;
  d.out = out;
  d.num_seqs = num_seqs;
  d.num_q_heads = num_q_heads;
  d.max_blocks = max_blocks;
  d.mode = pl.mode;
  d.partition_tokens = pl.partition_tokens;
  d.num_partitions = pl.num_partitions;
  d.chunks_per_wave = pl.chunks_per_wave;
  d.waves_per_unit = pl.waves_per_unit;
  d.scale = scale;
  if (pl.partial) {
    auto* ws = static_cast<uint8_t*>(workspace);
    d.part_m = reinterpret_cast<float*>(ws);
    d.part_l = reinterpret_cast<float*>(ws + pl.off_l);
    d.part_o = reinterpret_cast<float*>(ws + pl.off_o);
  }
  return d;
}

bool misaligned(const void* ptr, uintptr_t bytes) { return reinterpret_cast<uintptr_t>(ptr) % bytes != 0; }

// has_q: the call reads q (false when a multi-token batch has no query rows).
int check_decode_args(pa_pool* pool, int32_t layer, const void* q, const int32_t* tables,
                      const int32_t* lens, int32_t num_seqs, float scale, bool has_q = true) {
  int rc = check_bound(pool);
  if (rc) return rc;
  if ((rc = check_layer(pool, layer))) return rc;
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID, "scale is not finite");
  if (num_seqs > 0 && ((has_q && !q) || !tables || !lens)) return fail(PA_ERR_INVALID, "NULL device pointer");
  if (misaligned(q, 16)) return fail(PA_ERR_INVALID, "q must be 16-byte aligned");
  return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_last_error(void) { return g_last_error; }

int pa_pool_create(int32_t layers, int32_t kv_heads, int32_t head_dim, int32_t block_size,
                   int32_t dtype, int32_t num_blocks, pa_pool** out) {
  if (!out) return fail(PA_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (layers < 1 || kv_heads < 1) return fail(PA_ERR_INVALID, "layers and kv_heads must be >= 1");
  if (head_dim != pa::kHeadDimSmall && head_dim != pa::kHeadDimLarge)
    return fail(PA_ERR_INVALID, "head_dim %d unsupported (64 or 128)", head_dim);
  if (block_size != 8 && block_size != 16 && block_size != 32)
    return fail(PA_ERR_INVALID, "block_size %d unsupported (8, 16, 32)", block_size);
  if (dtype != PA_DTYPE_FP16 && dtype != PA_DTYPE_FP8_E4M3 && dtype != PA_DTYPE_INT8)
    return fail(PA_ERR_INVALID, "unknown dtype %d", dtype);
  if (num_blocks < 1 || static_cast<int64_t>(num_blocks) * block_size > 0x7FFFFFFF)
    return fail(PA_ERR_INVALID, "num_blocks %d out of range", num_blocks);
  try {
    *out = new pa_pool(layers, kv_heads, head_dim, block_size, dtype, num_blocks);
  } catch (const std::bad_alloc&) {
    return fail(PA_ERR_INVALID, "out of host memory");
  }
  return PA_OK;
}

int pa_pool_destroy(pa_pool* pool) {
  delete pool;
  return PA_OK;
}

int pa_pool_info_get(const pa_pool* p, pa_pool_info* out) {
  if (!p || !out) return fail(PA_ERR_INVALID, "NULL argument");
  out->layers = p->layers;
  out->kv_heads = p->kv_heads;
  out->head_dim = p->head_dim;
  out->block_size = p->block_size;
  out->dtype = p->dtype;
  out->num_blocks = p->num_blocks;
  out->elem_bytes = p->elem_bytes;
  out->bound = p->bound ? 1 : 0;
  out->tile_bytes = p->tile_bytes;
  out->kv_bytes = p->kv_bytes;
  out->total_bytes = p->total_bytes;
  // 1/sqrt(d): the square root and the division each rounded to fp32.
  out->softmax_scale = 1.0f / std::sqrt(static_cast<float>(p->head_dim));
  out->reserved = 0;
  return PA_OK;
}

int pa_pool_set_load_policy(pa_pool* p, int32_t policy) {
  if (!p) return fail(PA_ERR_INVALID, "pool is NULL");
  if (policy != PA_LOADS_AUTO && policy != PA_LOADS_STREAMING && policy != PA_LOADS_CACHED)
    return fail(PA_ERR_INVALID, "unknown load policy %d", policy);
  p->load_policy = policy;
  return PA_OK;
}

int pa_pool_load_policy(const pa_pool* p, int32_t* policy_out, int32_t* cached_now_out) {
  if (!p || !policy_out) return fail(PA_ERR_INVALID, "NULL argument");
  *policy_out = p->load_policy;
  if (cached_now_out) *cached_now_out = use_cached_loads(p) ? 1 : 0;
  return PA_OK;
}

int pa_pool_set_free_order(pa_pool* p, const int32_t* perm, int32_t n) {
  if (!p) return fail(PA_ERR_INVALID, "pool is NULL");
  if (p->bm.set_free_order(perm, n) != pa::BmStatus::kOk)
    return fail(PA_ERR_INVALID, "free order must be a permutation of 0..%d set before any allocation",
                p->num_blocks - 1);
  return PA_OK;
}

namespace {

int bind_pool(pa_pool* p, void* dev_base, const float* k_scales, const float* v_scales,
              const int32_t* k_zeros, const int32_t* v_zeros) {
  if (!p || !dev_base) return fail(PA_ERR_INVALID, "NULL argument");
  if (reinterpret_cast<uintptr_t>(dev_base) % 256 != 0)
    return fail(PA_ERR_INVALID, "device buffer must be 256-byte aligned");
  const size_t lh = static_cast<size_t>(p->layers) * p->kv_heads;
  // [6][layers][kv_heads]: k_scale, v_scale, k_inv, v_inv, k_zero, v_zero
  std::vector<float> sc(6 * lh, 1.0f);
  std::fill(sc.begin() + 4 * lh, sc.end(), 0.0f);
  if (p->dtype != PA_DTYPE_FP16) {
    if (!k_scales || !v_scales) return fail(PA_ERR_INVALID, "fp8 and int8 pools need k_scales and v_scales");
    for (size_t i = 0; i < lh; ++i) {
      const float ks = k_scales[i], vs = v_scales[i];
      if (!(std::isfinite(ks) && ks > 0.0f && std::isfinite(vs) && vs > 0.0f))
        return fail(PA_ERR_INVALID, "scale %zu is not a positive finite number", i);
      sc[i] = ks;
      sc[lh + i] = vs;
      sc[2 * lh + i] = 1.0f / ks;  // IEEE fp32 division, round to nearest even
      sc[3 * lh + i] = 1.0f / vs;
    }
  }
  if (p->dtype == PA_DTYPE_INT8) {
    if (!k_zeros || !v_zeros) return fail(PA_ERR_INVALID, "int8 pools need k_zeros and v_zeros");
    for (size_t i = 0; i < lh; ++i) {
      if (k_zeros[i] < -128 || k_zeros[i] > 127 || v_zeros[i] < -128 || v_zeros[i] > 127)
        return fail(PA_ERR_INVALID, "zero point %zu outside [-128, 127]", i);
      sc[4 * lh + i] = static_cast<float>(k_zeros[i]);
      sc[5 * lh + i] = static_cast<float>(v_zeros[i]);
    }
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
    p->num_cus = cus;
  auto* base = static_cast<uint8_t*>(dev_base);
  e = hipMemcpy(base + p->scales_offset, sc.data(), sc.size() * sizeof(float), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy(scales)");
  e = hipMemset(base + p->status_offset, 0, 256);
  if (e != hipSuccess) return hip_fail(e, "hipMemset(status)");
  pa::PoolGeom& g = p->geom;
  g.base = base;
  g.layers = p->layers;
  g.kv_heads = p->kv_heads;
  g.head_dim = p->head_dim;
  g.block_size = p->block_size;
  g.num_blocks = p->num_blocks;
  g.elem_bytes = p->elem_bytes;
  g.kind = p->dtype;  // PA_DTYPE_* values are the kernels' element kinds
  g.tile_bytes = p->tile_bytes;
  g.block_stride = p->tile_bytes * p->kv_heads;
  g.half_stride = g.block_stride * p->num_blocks;
  g.scales = reinterpret_cast<float*>(base + p->scales_offset);
  g.status = reinterpret_cast<uint32_t*>(base + p->status_offset);
  p->device = dev;
  // Set-up of pa_decode_noalloc's partials on this device (once per device;
  // a failure is reported by that call, not by the bind).
  p->scratch = scratch_on_current_device(dev, &p->scratch_err);
  p->bound = true;
  return PA_OK;
}

}  // namespace

int pa_pool_bind(pa_pool* p, void* dev_base, const float* k_scales, const float* v_scales) {
  if (p && p->dtype == PA_DTYPE_INT8)
    return fail(PA_ERR_INVALID, "int8 pools are bound with pa_pool_bind_int8 (they need zero points)");
  return bind_pool(p, dev_base, k_scales, v_scales, nullptr, nullptr);
}

int pa_pool_bind_int8(pa_pool* p, void* dev_base, const float* k_scales, const float* v_scales,
                      const int32_t* k_zeros, const int32_t* v_zeros) {
  if (p && p->dtype != PA_DTYPE_INT8) return fail(PA_ERR_INVALID, "pa_pool_bind_int8 needs an int8 pool");
  return bind_pool(p, dev_base, k_scales, v_scales, k_zeros, v_zeros);
}

int pa_seq_create(pa_pool* p, int32_t* seq_out) {
  if (!p || !seq_out) return fail(PA_ERR_INVALID, "NULL argument");
  *seq_out = p->bm.seq_create();
  return PA_OK;
}

int pa_seq_create_cached(pa_pool* p, const int32_t* tokens, int32_t n, int32_t* seq_out,
                         int32_t* cached_out, int32_t* slots_out) {
  if (!p || !seq_out || !cached_out) return fail(PA_ERR_INVALID, "NULL argument");
  if (n < 0) return fail(PA_ERR_INVALID, "n %d < 0", n);
  if (n > 0 && (!tokens || !slots_out)) return fail(PA_ERR_INVALID, "NULL argument");
  switch (p->bm.seq_create_cached(tokens, n, seq_out, cached_out, slots_out)) {
    case pa::BmStatus::kOk: return PA_OK;
    case pa::BmStatus::kNoBlocks: return fail(PA_ERR_NO_BLOCKS, "prompt of %d tokens does not fit", n);
    default: return fail(PA_ERR_INVALID, "invalid argument");
  }
}

int pa_alloc_tokens(pa_pool* p, int32_t seq, int32_t n_tokens, const int32_t* tokens, int32_t* slots_out,
                    int32_t* cow_out, void* stream) {
  if (!p) return fail(PA_ERR_INVALID, "pool is NULL");
  int32_t src = -1, dst = -1;
  const int rc = bm_status(p->bm.alloc(seq, n_tokens, slots_out, &src, &dst, tokens), seq);
  if (cow_out) {
    cow_out[0] = src;
    cow_out[1] = dst;
  }
  if (rc) return rc;
  if (src >= 0 && p->bound) {
    const hipError_t e = pa::launch_copy_blocks(p->geom, &src, &dst, 1, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "copy-on-write block copy");
  }
  return PA_OK;
}

int pa_alloc(pa_pool* p, int32_t seq, int32_t n_tokens, int32_t* slots_out, int32_t* cow_out,
             void* stream) {
  return pa_alloc_tokens(p, seq, n_tokens, nullptr, slots_out, cow_out, stream);
}

int pa_alloc_batch(pa_pool* p, const int32_t* seqs, const int32_t* n_tokens, int32_t count,
                   const int32_t* tokens, int32_t* slots_out, int32_t* cow_out, int32_t* done_out,
                   void* stream) {
  if (done_out) *done_out = 0;
  if (!p) return fail(PA_ERR_INVALID, "pool is NULL");
  if (count < 0 || (count > 0 && (!seqs || !n_tokens)))
    return fail(PA_ERR_INVALID, "bad arguments to pa_alloc_batch");
  int64_t total = 0;
  for (int32_t k = 0; k < count; ++k) {
    if (n_tokens[k] < 0) return fail(PA_ERR_INVALID, "n_tokens[%d] = %d < 0", k, n_tokens[k]);
    total += n_tokens[k];
  }
  if (total > 0 && !slots_out) return fail(PA_ERR_INVALID, "slots_out is NULL");
  // The appends in order, as pa_alloc does them; the copies of the whole
  // batch go to the device together afterwards.  Their order does not
  // matter: every copy's destination is a fresh block private to the
  // appending sequence, so no copy of the batch reads another's destination,
  // and no append frees a block.
  std::vector<int32_t> src, dst;
  int rc = PA_OK;
  int32_t k = 0;
  int64_t off = 0;
  for (; k < count; ++k) {
    int32_t s = -1, d = -1;
    rc = bm_status(p->bm.alloc(seqs[k], n_tokens[k], slots_out ? slots_out + off : nullptr, &s, &d,
                               tokens ? tokens + off : nullptr),
                   seqs[k]);
    if (cow_out) {
      cow_out[2 * k] = s;
      cow_out[2 * k + 1] = d;
    }
    if (rc) break;
    off += n_tokens[k];
    if (s >= 0) {
      src.push_back(s);
      dst.push_back(d);
    }
  }
  if (done_out) *done_out = k;
  if (!src.empty() && p->bound) {
    const hipError_t e = pa::launch_copy_blocks(p->geom, src.data(), dst.data(), static_cast<int>(src.size()),
                                                static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "copy-on-write block copies");
  }
  return rc;
}

int pa_fork(pa_pool* p, int32_t parent, int32_t* child_out) {
  if (!p || !child_out) return fail(PA_ERR_INVALID, "NULL argument");
  return bm_status(p->bm.fork(parent, child_out), parent);
}

int pa_free(pa_pool* p, int32_t seq) {
  if (!p) return fail(PA_ERR_INVALID, "pool is NULL");
  return bm_status(p->bm.free_seq(seq), seq);
}

int pa_seq_len(const pa_pool* p, int32_t seq, int32_t* len_out, int32_t* num_blocks_out) {
  if (!p) return fail(PA_ERR_INVALID, "pool is NULL");
  return bm_status(p->bm.seq_len(seq, len_out, num_blocks_out), seq);
}

int pa_block_tables(const pa_pool* p, const int32_t* seqs, int32_t n, int32_t max_blocks,
                    int32_t* tables_out, int32_t* lens_out) {
  if (!p || n < 0 || max_blocks < 0 || (n > 0 && (!seqs || !tables_out)))
    return fail(PA_ERR_INVALID, "bad arguments to pa_block_tables");
  for (int32_t i = 0; i < n; ++i) {
    int32_t len = 0;
    const pa::BmStatus s = p->bm.table_row(seqs[i], max_blocks,
                                           tables_out + static_cast<int64_t>(i) * max_blocks, &len);
    if (s == pa::BmStatus::kInvalid)
      return fail(PA_ERR_INVALID, "block table of sequence %d is longer than max_blocks %d", seqs[i], max_blocks);
    if (s != pa::BmStatus::kOk) return bm_status(s, seqs[i]);
    if (lens_out) lens_out[i] = len;
  }
  return PA_OK;
}

int pa_pool_stats(const pa_pool* p, pa_stats* out) {
  if (!p || !out) return fail(PA_ERR_INVALID, "NULL argument");
  out->num_blocks = p->num_blocks;
  out->free_blocks = p->bm.free_count();
  out->used_blocks = p->num_blocks - p->bm.free_count();
  out->shared_blocks = p->bm.shared_blocks();
  out->num_seqs = p->bm.live_seqs();
  out->cow_copies = p->bm.cow_copies();
  out->alloc_failures = p->bm.alloc_failures();
  out->cache_hits = p->bm.cache_hits();
  out->cache_misses = p->bm.cache_misses();
  out->cache_evictions = p->bm.cache_evictions();
  out->cached_blocks = p->bm.cached_blocks();
  return PA_OK;
}

int pa_refcounts(const pa_pool* p, int32_t* out) {
  if (!p || !out) return fail(PA_ERR_INVALID, "NULL argument");
  std::memcpy(out, p->bm.refcounts().data(), sizeof(int32_t) * p->num_blocks);
  return PA_OK;
}

int pa_free_queue(const pa_pool* p, int32_t* out, int32_t* n_out) {
  if (!p || !out || !n_out) return fail(PA_ERR_INVALID, "NULL argument");
  p->bm.free_queue(out);
  *n_out = static_cast<int32_t>(p->bm.free_count());
  return PA_OK;
}

int pa_write_kv(pa_pool* p, int32_t layer, const void* k_new, const void* v_new,
                const int32_t* slot_mapping, int32_t n_tokens, void* stream) {
  int rc = check_bound(p);
  if (rc) return rc;
  if ((rc = check_layer(p, layer))) return rc;
  if (n_tokens < 0) return fail(PA_ERR_INVALID, "n_tokens %d < 0", n_tokens);
  if (n_tokens > 0 && (!k_new || !v_new || !slot_mapping)) return fail(PA_ERR_INVALID, "NULL device pointer");
  if (misaligned(k_new, 16) || misaligned(v_new, 16))
    return fail(PA_ERR_INVALID, "k_new and v_new must be 16-byte aligned");
  const hipError_t e = pa::launch_write_kv(p->geom, layer, k_new, v_new, slot_mapping, n_tokens,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : hip_fail(e, "write_kv launch");
}

int pa_gather_kv(const pa_pool* p, int32_t layer, const int32_t* slot_mapping, int32_t n_tokens,
                 void* k_out, void* v_out, void* stream) {
  int rc = check_bound(p);
  if (rc) return rc;
  if ((rc = check_layer(p, layer))) return rc;
  if (n_tokens < 0) return fail(PA_ERR_INVALID, "n_tokens %d < 0", n_tokens);
  if (n_tokens > 0 && (!k_out || !v_out || !slot_mapping)) return fail(PA_ERR_INVALID, "NULL device pointer");
  const hipError_t e = pa::launch_gather_kv(p->geom, layer, slot_mapping, n_tokens, k_out, v_out,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : hip_fail(e, "gather_kv launch");
}

int pa_copy_blocks(pa_pool* p, const int32_t* src, const int32_t* dst, int32_t n, void* stream) {
  int rc = check_bound(p);
  if (rc) return rc;
  if (n < 0 || (n > 0 && (!src || !dst))) return fail(PA_ERR_INVALID, "bad copy list");
  for (int32_t i = 0; i < n; ++i) {
    if (src[i] < 0 || src[i] >= p->num_blocks || dst[i] < 0 || dst[i] >= p->num_blocks)
      return fail(PA_ERR_INVALID, "copy pair %d (%d -> %d) outside the pool", i, src[i], dst[i]);
  }
  const hipError_t e = pa::launch_copy_blocks(p->geom, src, dst, n, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : hip_fail(e, "copy_blocks launch");
}

int pa_decode_workspace_bytes(const pa_pool* p, int32_t num_seqs, int32_t num_q_heads,
                              int32_t max_blocks, int32_t partition_tokens, uint64_t* bytes_out) {
  if (!p || !bytes_out) return fail(PA_ERR_INVALID, "NULL argument");
  Plan pl;
  const int rc = make_plan(p, num_seqs, num_q_heads, max_blocks, partition_tokens, &pl);
  if (rc) return rc;
  *bytes_out = pl.partial ? pl.ws_bytes : 0;
  return PA_OK;
}

struct NewTokens {
  const void* k = nullptr;
  const void* v = nullptr;
  const int32_t* slots = nullptr;
};

static int run_decode(pa_pool* p, int32_t layer, const void* q, int32_t num_q_heads,
                      const int32_t* tables, int32_t max_blocks, const int32_t* lens,
                      int32_t num_seqs, const int32_t* order, float scale,
                      int32_t partition_tokens, void* out, void* workspace,
                      uint64_t workspace_bytes, void* stream, int mode,
                      const NewTokens& nt = NewTokens{}) {
  // mode 0: full decode, 1: partials only
  int rc = check_decode_args(p, layer, q, tables, lens, num_seqs, scale);
  if (rc) return rc;
  Plan pl;
  if ((rc = make_plan(p, num_seqs, num_q_heads, max_blocks, partition_tokens, &pl))) return rc;
  if (mode == 1 && !pl.partial) return fail(PA_ERR_INVALID, "pa_decode_partials needs partition_tokens > 0");
  if (mode == 0 && num_seqs > 0 && !out) return fail(PA_ERR_INVALID, "out is NULL");
  if (mode == 0 && misaligned(out, 8)) return fail(PA_ERR_INVALID, "out must be 8-byte aligned");
  if (pl.partial && misaligned(workspace, 16)) return fail(PA_ERR_INVALID, "workspace must be 16-byte aligned");
  // An empty batch needs no workspace (0 bytes, which may be NULL).
  if (pl.partial && pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes))
    return fail(PA_ERR_INVALID, "workspace of %llu bytes needed", static_cast<unsigned long long>(pl.ws_bytes));
  if (num_seqs == 0) return PA_OK;
  pa::DecodeLaunch d = make_launch(layer, q, num_q_heads, tables, max_blocks, lens, num_seqs,
                                   order, scale, pl, out, workspace);
  d.k_new = nt.k;
  d.v_new = nt.v;
  d.new_slots = nt.slots;
  d.cached_loads = use_cached_loads(p) ? 1 : 0;
  auto s = static_cast<hipStream_t>(stream);
  const bool rec = p->profiling && p->launches++ % p->every == 0 && p->n_records < p->max_records;
  hipEvent_t* ev = rec ? &p->ev[4 * static_cast<size_t>(p->n_records)] : nullptr;
  const bool reduced = pl.partial && mode == 0;
  hipError_t e = pa::launch_decode(p->geom, d, s, rec ? ev[0] : nullptr, rec ? ev[1] : nullptr);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  if (reduced) {
    e = pa::launch_lse_reduce(p->geom, d, s, rec ? ev[2] : nullptr, rec ? ev[3] : nullptr);
    if (e != hipSuccess) return hip_fail(e, "lse_reduce launch");
  }
  if (rec) {
    p->has_reduce[p->n_records] = reduced ? 1 : 0;
    ++p->n_records;
  }
  return PA_OK;
}

int pa_decode(pa_pool* p, int32_t layer, const void* q, int32_t num_q_heads,
              const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
              int32_t num_seqs, const int32_t* seq_order, float scale, int32_t partition_tokens,
              void* out, void* workspace, uint64_t workspace_bytes, void* stream) {
  return run_decode(p, layer, q, num_q_heads, block_tables, max_blocks, context_lens, num_seqs,
                    seq_order, scale, partition_tokens, out, workspace, workspace_bytes, stream, 0);
}

int pa_decode_noalloc(pa_pool* p, int32_t layer, const void* q, int32_t num_q_heads,
                      const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                      int32_t num_seqs, const int32_t* seq_order, float scale, int32_t partition_tokens,
                      void* out, void* stream) {
  int rc = check_bound(p);
  if (rc) return rc;
  Plan pl;
  if ((rc = make_plan(p, num_seqs, num_q_heads, max_blocks, partition_tokens, &pl))) return rc;
  void* ws = nullptr;
  uint64_t ws_bytes = 0;
  if (pl.partial && num_seqs > 0) {
    if (pl.ws_bytes > PA_NOALLOC_SCRATCH_BYTES)
      return fail(PA_ERR_INVALID,
                  "this launch needs %llu bytes of split-context partials, more than the %llu-byte "
                  "static scratch of pa_decode_noalloc (use pa_decode with a workspace, or fewer chunks)",
                  static_cast<unsigned long long>(pl.ws_bytes),
                  static_cast<unsigned long long>(PA_NOALLOC_SCRATCH_BYTES));
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev != p->device)
      return fail(PA_ERR_INVALID, "current device %d is not the pool's device %d", dev, p->device);
    if (!p->scratch) return hip_fail(p->scratch_err, "device address of the static scratch");
    ws = p->scratch;
    ws_bytes = PA_NOALLOC_SCRATCH_BYTES;
  }
  return run_decode(p, layer, q, num_q_heads, block_tables, max_blocks, context_lens, num_seqs,
                    seq_order, scale, partition_tokens, out, ws, ws_bytes, stream, 0);
}

int pa_write_kv_decode(pa_pool* p, int32_t layer, const void* k_new, const void* v_new,
                       const int32_t* slot_mapping, const void* q, int32_t num_q_heads,
                       const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                       int32_t num_seqs, const int32_t* seq_order, float scale,
                       int32_t partition_tokens, void* out, void* workspace,
                       uint64_t workspace_bytes, void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new || !slot_mapping))
    return fail(PA_ERR_INVALID, "k_new, v_new and slot_mapping are required");
  if (misaligned(k_new, 16) || misaligned(v_new, 16))
    return fail(PA_ERR_INVALID, "k_new and v_new must be 16-byte aligned");
  NewTokens nt;
  nt.k = k_new;
  nt.v = v_new;
  nt.slots = slot_mapping;
  return run_decode(p, layer, q, num_q_heads, block_tables, max_blocks, context_lens, num_seqs,
                    seq_order, scale, partition_tokens, out, workspace, workspace_bytes, stream, 0, nt);
}

}  // extern "C"

namespace {

// Copies n int32 from host memory to device memory `dst` on stream s through
// the pool's ring of pinned staging buffers (each reused once the event of
// the upload that last read it has completed, so the host can run several
// launches ahead of the device).
int upload_ints(pa_pool* p, void* dst, const int32_t* src, size_t n, hipStream_t s) {
  hipError_t e;
  pa_pool::Staging& st = p->mt_ring[p->mt_next];
  p->mt_next = (p->mt_next + 1) % pa_pool::kStagingRing;
  if (st.done) {
    e = hipEventSynchronize(st.done);  // this buffer's last upload has been read
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
  } else {
    e = hipEventCreateWithFlags(&st.done, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
  }
  if (st.cap < n) {
    if (st.host) (void)hipHostFree(st.host);
    st.host = nullptr;
    st.cap = 0;
    e = hipHostMalloc(reinterpret_cast<void**>(&st.host), n * sizeof(int32_t), hipHostMallocDefault);
    if (e != hipSuccess) return hip_fail(e, "hipHostMalloc(staging)");
    st.cap = n;
  }
  std::memcpy(st.host, src, n * sizeof(int32_t));
  e = hipMemcpyAsync(dst, st.host, n * sizeof(int32_t), hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(staging)");
  e = hipEventRecord(st.done, s);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  return PA_OK;
}

// Work items of a multi-token launch: for every sequence with query tokens,
// tiles of multi_token_tile(G) tokens, the later tiles (which see more keys)
// first within a sequence; wide and narrow tiles alternate.  Returns the number of items, or -1 after fail() for a bad
// query_start.
int64_t multi_token_items(const pa_pool* p, const int32_t* query_start, int32_t num_seqs, int32_t group,
                          std::vector<int32_t>* items) {
  if (num_seqs < 0) return fail(PA_ERR_INVALID, "num_seqs %d < 0", num_seqs), -1;
  if (num_seqs > 0 && !query_start) return fail(PA_ERR_INVALID, "query_start is NULL"), -1;
  if (num_seqs > 0 && query_start[0] != 0) return fail(PA_ERR_INVALID, "query_start[0] must be 0"), -1;
  const int tq = pa::multi_token_tile(group);
  int64_t n_items = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int64_t n_i = static_cast<int64_t>(query_start[i + 1]) - query_start[i];
    if (n_i < 0) return fail(PA_ERR_INVALID, "query_start decreases at sequence %d", i), -1;
    n_items += (n_i + tq - 1) / tq;
  }
  if (items) {
    items->clear();
    items->reserve(static_cast<size_t>(4 * n_items));
    // Narrow items (decode tokens: HBM-bound) and wide ones (prefill tiles:
    // more query tokens than one wave takes, MFMA-bound) alternate, so that
    // both kinds run on every CU at once and the matrix cores and the memory
    // system work together (with the prefill tiles first the two kinds ran
    // one after the other).
    std::vector<int32_t> wide_items, short_items;
    const int tw = pa::multi_token_wave_tile(group);
    for (int32_t i = 0; i < num_seqs; ++i) {
      const int32_t n_i = query_start[i + 1] - query_start[i];
      for (int32_t t = (n_i + tq - 1) / tq - 1; t >= 0; --t) {
        const int32_t nq = std::min<int32_t>(n_i - t * tq, tq);
        std::vector<int32_t>& dst = nq > tw ? wide_items : short_items;
        dst.push_back(i);
        dst.push_back(t * tq);
        dst.push_back(query_start[i] + t * tq);
        dst.push_back(n_i);
      }
    }
    size_t a = 0, b = 0;
    while (a < wide_items.size() || b < short_items.size()) {
      if (b < short_items.size()) {
        items->insert(items->end(), short_items.begin() + b, short_items.begin() + b + 4);
        b += 4;
      }
      if (a < wide_items.size()) {
        items->insert(items->end(), wide_items.begin() + a, wide_items.begin() + a + 4);
        a += 4;
      }
    }
  }
  (void)p;
  return n_items;
}

}  // namespace

extern "C" {

int pa_multi_token_workspace_bytes(const pa_pool* p, const int32_t* query_start, int32_t num_seqs,
                                   int32_t num_q_heads, uint64_t* bytes_out) {
  if (!p || !bytes_out) return fail(PA_ERR_INVALID, "NULL argument");
  if (num_q_heads < 1 || num_q_heads % p->kv_heads != 0 || num_q_heads / p->kv_heads > 32)
    return fail(PA_ERR_INVALID, "num_q_heads %d must be a multiple of kv_heads %d with a group of at most 32",
                num_q_heads, p->kv_heads);
  const int64_t n = multi_token_items(p, query_start, num_seqs, num_q_heads / p->kv_heads, nullptr);
  if (n < 0) return PA_ERR_INVALID;
  *bytes_out = static_cast<uint64_t>(n) * 16;
  return PA_OK;
}

int pa_multi_token_attention(pa_pool* p, int32_t layer, const void* q, int32_t num_q_heads,
                             const int32_t* query_start, const int32_t* block_tables, int32_t max_blocks,
                             const int32_t* context_lens, int32_t num_seqs, float scale, void* out,
                             void* workspace, uint64_t workspace_bytes, void* stream) {
  // With no query rows at all (every n_i = 0) q and out hold nothing and
  // may be NULL.
  const bool no_rows = num_seqs > 0 && query_start && query_start[num_seqs] == 0;
  int rc = check_decode_args(p, layer, q, block_tables, context_lens, num_seqs, scale, !no_rows);
  if (rc) return rc;
  if (scale == 0.0f) return fail(PA_ERR_INVALID, "scale must be nonzero");
  if (num_q_heads < 1 || num_q_heads % p->kv_heads != 0 || num_q_heads / p->kv_heads > 32)
    return fail(PA_ERR_INVALID, "num_q_heads %d must be a multiple of kv_heads %d with a group of at most 32",
                num_q_heads, p->kv_heads);
  if (max_blocks < 1 || static_cast<int64_t>(max_blocks) * p->block_size > 0x7FFFFFFF)
    return fail(PA_ERR_INVALID, "max_blocks %d out of range", max_blocks);
  std::vector<int32_t> items;
  const int64_t n_items = multi_token_items(p, query_start, num_seqs, num_q_heads / p->kv_heads, &items);
  if (n_items < 0) return PA_ERR_INVALID;
  if (n_items == 0) return PA_OK;
  if (!out) return fail(PA_ERR_INVALID, "out is NULL");
  if (misaligned(out, 8)) return fail(PA_ERR_INVALID, "out must be 8-byte aligned");
  const uint64_t need = static_cast<uint64_t>(n_items) * 16;
  if (!workspace || workspace_bytes < need || misaligned(workspace, 16))
    return fail(PA_ERR_INVALID, "a 16-byte aligned workspace of %llu bytes is needed",
                static_cast<unsigned long long>(need));
  if (n_items * p->kv_heads > 0x7FFFFFFF) return fail(PA_ERR_INVALID, "too many query tiles");
  auto s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if ((rc = upload_ints(p, workspace, items.data(), items.size(), s))) return rc;
  pa::DecodeLaunch d{};
  d.layer = layer;
  d.q = q;
  d.tables = block_tables;
  d.lens = context_lens;
  d.out = out;
  d.num_seqs = num_seqs;
  d.num_q_heads = num_q_heads;
  d.max_blocks = max_blocks;
  d.scale = scale;
  d.work = static_cast<const int32_t*>(workspace);
  d.num_items = static_cast<int>(n_items);
  const bool rec = p->profiling && p->launches++ % p->every == 0 && p->n_records < p->max_records;
  hipEvent_t* ev = rec ? &p->ev[4 * static_cast<size_t>(p->n_records)] : nullptr;
  e = pa::launch_multi_token(p->geom, d, s, rec ? ev[0] : nullptr, rec ? ev[1] : nullptr);
  if (e != hipSuccess) return hip_fail(e, "multi-token launch");
  if (rec) {
    p->has_reduce[p->n_records] = 0;
    ++p->n_records;
  }
  return PA_OK;
}

int pa_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, void* stream) {
  if (bytes == 0) return PA_OK;
  if (!buf || !sink) return fail(PA_ERR_INVALID, "NULL device pointer");
  if (bytes % 16 != 0 || misaligned(buf, 16))
    return fail(PA_ERR_INVALID, "bytes must be a multiple of 16 and buf 16-byte aligned");
  const hipError_t e = pa::launch_stream_read(buf, bytes, sink, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : hip_fail(e, "stream_read launch");
}

int pa_order_longest_first(const int32_t* lens, int32_t n, int32_t* order_out) {
  if (n < 0) return fail(PA_ERR_INVALID, "n %d < 0", n);
  if (n > 0 && (!lens || !order_out)) return fail(PA_ERR_INVALID, "NULL argument");
  for (int32_t i = 0; i < n; ++i) order_out[i] = i;
  std::stable_sort(order_out, order_out + n, [lens](int32_t a, int32_t b) { return lens[a] > lens[b]; });
  return PA_OK;
}

int pa_decode_partials(pa_pool* p, int32_t layer, const void* q, int32_t num_q_heads,
                       const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                       int32_t num_seqs, const int32_t* seq_order, float scale,
                       int32_t partition_tokens, void* workspace, uint64_t workspace_bytes,
                       void* stream) {
  if (partition_tokens <= 0) return fail(PA_ERR_INVALID, "pa_decode_partials needs partition_tokens > 0");
  return run_decode(p, layer, q, num_q_heads, block_tables, max_blocks, context_lens, num_seqs,
                    seq_order, scale, partition_tokens, nullptr, workspace, workspace_bytes, stream, 1);
}

int pa_lse_reduce(pa_pool* p, const void* workspace, uint64_t workspace_bytes,
                  const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                  int32_t max_blocks, int32_t partition_tokens, void* out, void* stream) {
  int rc = check_bound(p);
  if (rc) return rc;
  if (partition_tokens <= 0) return fail(PA_ERR_INVALID, "pa_lse_reduce needs partition_tokens > 0");
  Plan pl;
  if ((rc = make_plan(p, num_seqs, num_q_heads, max_blocks, partition_tokens, &pl))) return rc;
  if (num_seqs == 0) return PA_OK;
  if (!workspace || workspace_bytes < pl.ws_bytes || !out || !context_lens)
    return fail(PA_ERR_INVALID, "workspace of %llu bytes, out and context_lens needed",
                static_cast<unsigned long long>(pl.ws_bytes));
  if (misaligned(workspace, 16) || misaligned(out, 8))
    return fail(PA_ERR_INVALID, "the workspace must be 16-byte and out 8-byte aligned, as for pa_decode");
  const pa::DecodeLaunch d = make_launch(0, nullptr, num_q_heads, nullptr, max_blocks, context_lens,
                                         num_seqs, nullptr, 1.0f, pl, out, const_cast<void*>(workspace));
  const hipError_t e = pa::launch_lse_reduce(p->geom, d, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : hip_fail(e, "lse_reduce launch");
}

int pa_device_status(pa_pool* p, uint32_t* flags_out, int32_t clear, void* stream) {
  int rc = check_bound(p);
  if (rc) return rc;
  if (!flags_out) return fail(PA_ERR_INVALID, "flags_out is NULL");
  auto s = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, p->geom.status, sizeof(v), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "reading device status");
  *flags_out = v;
  if (clear) {
    const uint32_t zero = 0;
    e = hipMemcpyAsync(p->geom.status, &zero, sizeof(zero), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "clearing device status");
  }
  return PA_OK;
}

int pa_profile_begin(pa_pool* p, int32_t max_launches, int32_t every) {
  int rc = check_bound(p);
  if (rc) return rc;
  if (max_launches < 1) return fail(PA_ERR_INVALID, "max_launches must be >= 1");
  if (every < 1) return fail(PA_ERR_INVALID, "every must be >= 1");
  const size_t need = 4ull * max_launches;
  while (p->ev.size() < need) {
    hipEvent_t e;
    // Agent-scope release: recording needs no system-wide cache write-back.
    const hipError_t err = hipEventCreateWithFlags(&e, hipEventDisableSystemFence);
    if (err != hipSuccess) return hip_fail(err, "hipEventCreate");
    p->ev.push_back(e);
  }
  p->has_reduce.assign(max_launches, 0);
  p->max_records = max_launches;
  p->n_records = 0;
  p->every = every;
  p->launches = 0;
  p->profiling = true;
  return PA_OK;
}

int pa_profile_end(pa_pool* p, pa_profile* out) {
  int rc = check_bound(p);
  if (rc) return rc;
  if (!out) return fail(PA_ERR_INVALID, "out is NULL");
  pa_profile r{};
  for (int32_t i = 0; i < p->n_records; ++i) {
    const hipEvent_t* ev = &p->ev[4 * static_cast<size_t>(i)];
    hipError_t e = hipEventSynchronize(ev[p->has_reduce[i] ? 3 : 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, ev[0], ev[1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    r.decode_ms += ms;
    ++r.decode_launches;
    if (p->has_reduce[i]) {
      e = hipEventElapsedTime(&ms, ev[2], ev[3]);
      if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
      r.reduce_ms += ms;
      ++r.reduce_launches;
    }
  }
  p->profiling = false;
  p->n_records = 0;
  *out = r;
  return PA_OK;
}

}  // extern "C"

namespace {

// Workspace of a shared-prefix decode: the pieces' partials (m, l, o of
// every slot and query head), then the uploaded int32 tail: starts[S],
// slot0[S], members[S], the sequences with private pieces (S entries, the
// first n_private used) and the shared items (4 ints each).
struct SharedLayout {
  uint64_t off_l, off_o, off_c, bytes;
};

SharedLayout shared_layout(const pa_pool* p, int32_t num_seqs, int32_t num_q_heads, int64_t n_items,
                           int64_t n_slots) {
  const uint64_t rows = static_cast<uint64_t>(n_slots) * num_q_heads;
  SharedLayout L;
  L.off_l = align_up(std::max<uint64_t>(rows, 1) * 4, 256);
  L.off_o = L.off_l + align_up(std::max<uint64_t>(rows, 1) * 4, 256);
  L.off_c = L.off_o + align_up(std::max<uint64_t>(rows, 1) * p->head_dim * 4, 256);
  L.bytes = L.off_c + align_up((4ull * num_seqs + 4ull * n_items) * 4, 256);
  return L;
}

// Groups whose members have at most this many tokens of their own past the
// shared run are folded: one workgroup per member run streams the shared
// tokens and then each member's own tokens (one wave per member), so those
// members need neither a private piece nor a merge.  Measured on MI355X with
// beam search (32 groups of 5 beams, 2040 shared tokens, 4 to 70 own).
constexpr int64_t kFoldTokens = 128;

struct SharedTail {
  std::vector<int32_t> ints;  // starts, slot0, members, private sequences, items
  int64_t n_items = 0, n_slots = 0, n_private = 0;
  int32_t chunk = 0;
  bool reread = false;  // some chunk is read by several items (a group of more than 32 / G members)
};

// Checks the groups of a shared-prefix decode, picks the shared chunk length
// and builds the int32 tail.  Returns PA_OK or the status of fail().
int shared_groups_tail(const pa_pool* p, int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks,
                       const int32_t* members, const int32_t* group_start, const int32_t* shared_blocks,
                       int32_t num_groups, int32_t chunk_tokens, const int32_t* lens, SharedTail* out) {
  if (num_groups < 0 || num_seqs < 0) return fail(PA_ERR_INVALID, "num_groups and num_seqs must be >= 0");
  if ((num_seqs > 0 && !members) || ((num_seqs > 0 || num_groups > 0) && (!group_start || !shared_blocks)))
    return fail(PA_ERR_INVALID, "members, group_start and shared_blocks are required");
  // group_start must be a non-decreasing run from 0 to num_seqs before any
  // group's members are read.
  if (num_seqs > 0 || num_groups > 0) {
    if (group_start[0] != 0 || group_start[num_groups] != num_seqs)
      return fail(PA_ERR_INVALID, "group_start must run from 0 to num_seqs");
    for (int32_t g = 0; g < num_groups; ++g)
      if (group_start[g + 1] < group_start[g]) return fail(PA_ERR_INVALID, "group_start decreases at group %d", g);
  }
  if (chunk_tokens < 0 || chunk_tokens % 64 != 0)
    return fail(PA_ERR_INVALID, "chunk_tokens %d must be 0 (library choice) or a positive multiple of 64",
                chunk_tokens);
  const int group = num_q_heads / p->kv_heads;
  const int per_item = group >= 32 ? 1 : 32 / group;  // members whose heads fit 32 columns
  const size_t S = static_cast<size_t>(num_seqs);
  std::vector<char> seen(S, 0);
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int32_t m = members[i];
    if (m < 0 || m >= num_seqs || seen[m]) return fail(PA_ERR_INVALID, "members must be a permutation");
    seen[m] = 1;
  }
  // Shared runs, which groups fold (with the host lengths), and the work
  // items of one chunk per unfolded group.
  std::vector<char> fold(static_cast<size_t>(num_groups), 0);
  int64_t base_items = 0, max_ts = 0;
  for (int32_t g = 0; g < num_groups; ++g) {
    const int32_t a = group_start[g], b = group_start[g + 1];
    const int64_t ts = static_cast<int64_t>(shared_blocks[g]) * p->block_size;
    if (shared_blocks[g] < 0 || shared_blocks[g] > max_blocks || ts % 16 != 0)
      return fail(PA_ERR_INVALID, "shared_blocks[%d] = %d: not a multiple of 16 tokens inside the table", g,
                  shared_blocks[g]);
    if (ts == 0) continue;
    bool f = lens != nullptr;
    for (int32_t i = a; f && i < b; ++i) {
      const int64_t own = static_cast<int64_t>(lens[members[i]]) - ts;
      f = own >= 1 && own <= kFoldTokens;
    }
    fold[g] = f;
    if (f) continue;
    base_items += (b - a + per_item - 1) / per_item;
    max_ts = std::max(max_ts, ts);
  }
  // Chunk length: enough shared workgroups for one per CU (the second slot
  // of each CU runs the private pieces beside them), in whole 64-token runs
  // of the four waves, at least 256 tokens.  Measured on MI355X (beam
  // search, 32 groups of 5 beams over 2040 shared tokens, 8 KV heads): 69.0
  // us per launch with one 2048-token chunk per group, 72.1 with 1024, 79.0
  // with 512.
  int64_t chunk = chunk_tokens;
  if (chunk == 0) {
    chunk = std::max<int64_t>(max_ts, 64);
    if (base_items > 0) {
      const int64_t target = p->num_cus;
      const int64_t parts = (target + base_items * p->kv_heads - 1) / (base_items * p->kv_heads);
      chunk = align_up(static_cast<uint64_t>((max_ts + parts - 1) / parts), 64);
      chunk = std::max<int64_t>(std::min<int64_t>(chunk, align_up(static_cast<uint64_t>(max_ts), 64)), 256);
    }
  }
  if (chunk > 0x7FFFFFFF) return fail(PA_ERR_INVALID, "chunk_tokens out of range");
  out->chunk = static_cast<int32_t>(chunk);
  std::vector<int32_t>& t = out->ints;
  t.assign(4 * S, 0);
  int32_t* starts = t.data();
  int32_t* slot0 = starts + S;
  int32_t* mem_out = slot0 + S;
  int32_t* priv = mem_out + S;
  for (size_t i = 0; i < S; ++i) slot0[i] = -1;
  for (int32_t i = 0; i < num_seqs; ++i) mem_out[i] = members[i];
  int64_t slots = 0, n_items = 0, n_priv = 0;
  std::vector<int32_t> items;
  for (int32_t g = 0; g < num_groups; ++g) {
    const int32_t a = group_start[g], b = group_start[g + 1];
    const int64_t ts = static_cast<int64_t>(shared_blocks[g]) * p->block_size;
    if (ts == 0) {
      for (int32_t i = a; i < b; ++i) priv[n_priv++] = members[i];
      continue;
    }
    if (b - a > per_item) out->reread = true;
    if (fold[g]) {
      for (int32_t i = a; i < b; ++i) starts[members[i]] = static_cast<int32_t>(ts);
      for (int32_t i = a; i < b; i += per_item) {
        items.push_back(i);
        items.push_back(std::min<int32_t>(per_item, b - i));
        items.push_back(static_cast<int32_t>(ts));
        items.push_back(-1);
        ++n_items;
      }
      continue;
    }
    for (int32_t i = a; i < b; ++i) priv[n_priv++] = members[i];
    const int64_t chunks = (ts + chunk - 1) / chunk;
    for (int32_t i = a; i < b; ++i) {
      starts[members[i]] = static_cast<int32_t>(ts);
      slot0[members[i]] = static_cast<int32_t>(slots);
      slots += chunks + 1;
      if (slots > 0x7FFFFFFF / std::max(num_q_heads, 1)) return fail(PA_ERR_INVALID, "too many partial slots");
    }
    for (int64_t c = 0; c < chunks; ++c) {
      for (int32_t i = a; i < b; i += per_item) {
        items.push_back(i);
        items.push_back(std::min<int32_t>(per_item, b - i));
        items.push_back(static_cast<int32_t>(ts));
        items.push_back(static_cast<int32_t>(c));
        ++n_items;
      }
    }
  }
  if ((n_items + num_seqs) * p->kv_heads > 0x7FFFFFFF) return fail(PA_ERR_INVALID, "too many workgroups");
  if (lens) {
    // Longest own part first, as pa_order_longest_first does for the plain
    // decode: the last workgroups to start are then the short ones.
    std::stable_sort(priv, priv + n_priv, [&](int32_t x, int32_t y) {
      return static_cast<int64_t>(lens[x]) - starts[x] > static_cast<int64_t>(lens[y]) - starts[y];
    });
  }
  t.insert(t.end(), items.begin(), items.end());
  out->n_items = n_items;
  out->n_slots = slots;
  out->n_private = n_priv;
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_shared_prefix_groups(const pa_pool* p, const int32_t* tables, const int32_t* lens, int32_t n,
                            int32_t max_blocks, int32_t min_shared_tokens, int32_t* members_out,
                            int32_t* group_start_out, int32_t* shared_blocks_out, int32_t* num_groups_out) {
  if (!p || n < 0 || max_blocks < 1 || !num_groups_out ||
      (n > 0 && (!tables || !lens || !members_out || !group_start_out || !shared_blocks_out)))
    return fail(PA_ERR_INVALID, "bad arguments to pa_shared_prefix_groups");
  const int32_t bs = p->block_size;
  const int32_t quantum = bs >= 16 ? 1 : 16 / bs;  // blocks per 16 tokens
  // Candidates: sequences with at least one 16-token run of full blocks
  // before the block of their last token, keyed by their first block.
  std::vector<int32_t> order;
  std::vector<int32_t> singles;
  for (int32_t i = 0; i < n; ++i) {
    const int64_t full = lens[i] >= 1 ? (static_cast<int64_t>(lens[i]) - 1) / bs : 0;
    if (full >= quantum && tables[static_cast<int64_t>(i) * max_blocks] >= 0) order.push_back(i);
    else singles.push_back(i);
  }
  std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
    return tables[static_cast<int64_t>(x) * max_blocks] < tables[static_cast<int64_t>(y) * max_blocks];
  });
  int32_t ng = 0, pos = 0;
  group_start_out[0] = 0;
  auto emit = [&](const int32_t* seqs, int32_t cnt, int32_t shared) {
    for (int32_t k = 0; k < cnt; ++k) members_out[pos++] = seqs[k];
    shared_blocks_out[ng] = shared;
    group_start_out[++ng] = pos;
  };
  for (size_t a = 0; a < order.size();) {
    size_t b = a + 1;
    const int32_t* row0 = tables + static_cast<int64_t>(order[a]) * max_blocks;
    while (b < order.size() && tables[static_cast<int64_t>(order[b]) * max_blocks] == row0[0]) ++b;
    // Longest common run of block ids, inside every member's full blocks
    // that precede its last token, rounded down to 16 tokens.
    int64_t k = max_blocks;
    for (size_t i = a; i < b; ++i) k = std::min<int64_t>(k, (static_cast<int64_t>(lens[order[i]]) - 1) / bs);
    for (size_t i = a + 1; i < b && k > 0; ++i) {
      const int32_t* row = tables + static_cast<int64_t>(order[i]) * max_blocks;
      int64_t c = 0;
      while (c < k && row[c] == row0[c]) ++c;
      k = c;
    }
    k -= k % quantum;
    if (b - a >= 2 && k * bs >= min_shared_tokens && k > 0) {
      emit(order.data() + a, static_cast<int32_t>(b - a), static_cast<int32_t>(k));
    } else {
      for (size_t i = a; i < b; ++i) emit(&order[i], 1, 0);
    }
    a = b;
  }
  for (int32_t i : singles) emit(&i, 1, 0);
  *num_groups_out = ng;
  return PA_OK;
}

int pa_decode_shared_prefix_workspace_bytes(const pa_pool* p, int32_t num_seqs, int32_t num_q_heads,
                                            const int32_t* members, const int32_t* group_start,
                                            const int32_t* shared_blocks, int32_t num_groups,
                                            int32_t max_blocks, int32_t chunk_tokens, const int32_t* lens,
                                            uint64_t* bytes_out) {
  if (!p || !bytes_out || num_seqs < 0) return fail(PA_ERR_INVALID, "bad arguments");
  if (num_q_heads < 1 || num_q_heads % p->kv_heads != 0 || num_q_heads / p->kv_heads > 32)
    return fail(PA_ERR_INVALID, "num_q_heads %d must be a multiple of kv_heads %d with a group of at most 32",
                num_q_heads, p->kv_heads);
  SharedTail t;
  int rc = shared_groups_tail(p, num_seqs, num_q_heads, max_blocks, members, group_start, shared_blocks,
                              num_groups, chunk_tokens, lens, &t);
  if (rc) return rc;
  *bytes_out = num_seqs == 0 ? 0 : shared_layout(p, num_seqs, num_q_heads, t.n_items, t.n_slots).bytes;
  return PA_OK;
}

int pa_shared_prefix_plan(pa_pool* p, int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks,
                          const int32_t* members, const int32_t* group_start, const int32_t* shared_blocks,
                          int32_t num_groups, int32_t chunk_tokens, const int32_t* lens, void* workspace,
                          uint64_t workspace_bytes, void* stream, pa_shared_plan* plan) {
  int rc = check_bound(p);
  if (rc) return rc;
  if (!plan || num_seqs < 0) return fail(PA_ERR_INVALID, "bad arguments to pa_shared_prefix_plan");
  *plan = pa_shared_plan{};
  if (num_q_heads < 1 || num_q_heads % p->kv_heads != 0 || num_q_heads / p->kv_heads > 32)
    return fail(PA_ERR_INVALID, "num_q_heads %d must be a multiple of kv_heads %d with a group of at most 32",
                num_q_heads, p->kv_heads);
  if (max_blocks < 1 || static_cast<int64_t>(max_blocks) * p->block_size > 0x7FFFFFFF)
    return fail(PA_ERR_INVALID, "max_blocks %d out of range", max_blocks);
  SharedTail t;
  if ((rc = shared_groups_tail(p, num_seqs, num_q_heads, max_blocks, members, group_start, shared_blocks,
                               num_groups, chunk_tokens, lens, &t)))
    return rc;
  if (num_seqs > 0) {
    const SharedLayout L = shared_layout(p, num_seqs, num_q_heads, t.n_items, t.n_slots);
    if (!workspace || workspace_bytes < L.bytes || misaligned(workspace, 16))
      return fail(PA_ERR_INVALID, "a 16-byte aligned workspace of %llu bytes is needed",
                  static_cast<unsigned long long>(L.bytes));
    auto* ints = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(workspace) + L.off_c);
    if ((rc = upload_ints(p, ints, t.ints.data(), t.ints.size(), static_cast<hipStream_t>(stream)))) return rc;
  }
  plan->pool = p;
  plan->num_seqs = num_seqs;
  plan->num_q_heads = num_q_heads;
  plan->max_blocks = max_blocks;
  plan->num_items = static_cast<int32_t>(t.n_items);
  plan->num_slots = static_cast<int32_t>(t.n_slots);
  plan->num_private = static_cast<int32_t>(t.n_private);
  plan->chunk_tokens = t.chunk;
  plan->flags = t.reread ? PA_SHARED_REREAD : 0;
  plan->workspace = workspace;
  plan->workspace_bytes = workspace_bytes;
  return PA_OK;
}

int pa_decode_shared_prefix(pa_pool* p, int32_t layer, const pa_shared_plan* plan, const void* q,
                            const int32_t* block_tables, const int32_t* context_lens, const void* k_new,
                            const void* v_new, const int32_t* slot_mapping, float scale, void* out,
                            void* stream) {
  if (!plan || plan->pool != p) return fail(PA_ERR_INVALID, "the plan was not made for this pool");
  const int32_t num_seqs = plan->num_seqs, num_q_heads = plan->num_q_heads, max_blocks = plan->max_blocks;
  int rc = check_decode_args(p, layer, q, block_tables, context_lens, num_seqs, scale);
  if (rc) return rc;
  if (scale == 0.0f) return fail(PA_ERR_INVALID, "scale must be nonzero");
  const bool fused = k_new || v_new || slot_mapping;
  if (fused && (!k_new || !v_new || !slot_mapping))
    return fail(PA_ERR_INVALID, "k_new, v_new and slot_mapping go together");
  if (misaligned(k_new, 16) || misaligned(v_new, 16))
    return fail(PA_ERR_INVALID, "k_new and v_new must be 16-byte aligned");
  if (num_seqs == 0) return PA_OK;
  if (!out || misaligned(out, 8)) return fail(PA_ERR_INVALID, "out must be non-NULL and 8-byte aligned");
  if (plan->num_items < 0 || plan->num_slots < 0 || plan->chunk_tokens < 64 || plan->chunk_tokens % 64 != 0 ||
      plan->num_private < 0 || plan->num_private > num_seqs)
    return fail(PA_ERR_INVALID, "the plan is not one pa_shared_prefix_plan made");
  const SharedLayout L = shared_layout(p, num_seqs, num_q_heads, plan->num_items, plan->num_slots);
  if (!plan->workspace || plan->workspace_bytes < L.bytes)
    return fail(PA_ERR_INVALID, "the plan's workspace is too small");
  auto s = static_cast<hipStream_t>(stream);
  auto* ws = static_cast<uint8_t*>(plan->workspace);
  auto* ints = reinterpret_cast<int32_t*>(ws + L.off_c);
  const size_t S = static_cast<size_t>(num_seqs);
  pa::DecodeLaunch d{};
  d.layer = layer;
  d.q = q;
  d.tables = block_tables;
  d.lens = context_lens;
  d.out = out;
  d.num_seqs = num_seqs;
  d.num_q_heads = num_q_heads;
  d.max_blocks = max_blocks;
  d.mode = kModePrivate;
  d.partition_tokens = static_cast<int>(align_up(static_cast<uint64_t>(max_blocks) * p->block_size, 16));
  d.num_partitions = 1;
  d.chunks_per_wave = 1;
  d.waves_per_unit = 1;
  d.scale = scale;
  // The shared pieces read each shared block once; ordinary (cached) loads
  // only where several items of a group read the same chunk, nontemporal
  // ones otherwise (beams: 46.0 against 52.2 us for their shared pieces).
  d.cached_loads = (plan->flags & PA_SHARED_REREAD) ? 1 : 0;
  d.part_m = reinterpret_cast<float*>(ws);
  d.part_l = reinterpret_cast<float*>(ws + L.off_l);
  d.part_o = reinterpret_cast<float*>(ws + L.off_o);
  d.starts = ints;
  d.slot0 = d.starts + S;
  d.members = d.slot0 + S;
  d.order = d.members + S;  // the sequences with private pieces
  d.work = d.order + S;
  d.num_items = plan->num_items;
  d.sp_chunk = plan->chunk_tokens;
  d.sp_slots = plan->num_slots;
  d.sp_private = plan->num_private;
  if (fused) {
    d.k_new = k_new;
    d.v_new = v_new;
    d.new_slots = slot_mapping;
  }
  const bool rec = p->profiling && p->launches++ % p->every == 0 && p->n_records < p->max_records;
  hipEvent_t* ev = rec ? &p->ev[4 * static_cast<size_t>(p->n_records)] : nullptr;
  const hipError_t e = pa::launch_shared_prefix(p->geom, d, s, rec ? ev[0] : nullptr, rec ? ev[1] : nullptr);
  if (e != hipSuccess) return hip_fail(e, "shared-prefix launch");
  if (rec) {
    p->has_reduce[p->n_records] = 0;
    ++p->n_records;
  }
  return PA_OK;
}

}  // extern "C"
