// C ABI of libattn.so: argument validation, launch-shape selection, error reporting.
// Every entry point validates on the host before touching the HIP runtime, returns a
// status code and never lets a C++ exception escape.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/attn.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

attn_status_t fail(attn_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

attn_status_t ok() {
  g_last_error.clear();
  return ATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool valid_d(int d) { return d == 64 || d == 128 || d == 256; }

attn_status_t device_ready() {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return fail(ATTN_ERR_NO_DEVICE, "no HIP device is available");
  }
  return ATTN_OK;
}

attn_status_t launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(ATTN_ERR_LAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

constexpr int64_t kMaxGridYZ = 65535;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Output rounding: any of the three modes for bf16, RTNE only for fp16, ignored for fp32.
attn_status_t check_round(int32_t mode, int32_t o_dtype) {
  if (mode != ATTN_ROUND_RTNE && mode != ATTN_ROUND_RTNA && mode != ATTN_ROUND_RTZ)
    return fail(ATTN_ERR_INVALID_ARG, "o_round must be ATTN_ROUND_RTNE, ATTN_ROUND_RTNA or ATTN_ROUND_RTZ");
  if (o_dtype == ATTN_F16 && mode != ATTN_ROUND_RTNE)
    return fail(ATTN_ERR_UNSUPPORTED, "fp16 outputs are rounded to nearest even only");
  return ATTN_OK;
}

// Balanced decode plan in the workspace: {total, chunk, nwk} (256 bytes), prefix [B + 1],
// start [kMaxStreamWG].
constexpr int kMaxStreamWG = 1024;   // workgroups per KV head of the balanced split kernel
size_t plan_bytes(int64_t batch) {
  return 256 + align256((size_t)(batch + 1) * sizeof(int32_t)) + align256(kMaxStreamWG * sizeof(int32_t));
}

// Compute units of the current device (cached per device; callers may race, and all of
// them store the same value).
int device_cus() {
  static std::atomic<int> cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    if (const int c = cache[dev].load(std::memory_order_relaxed); c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
  if (dev < 64 && n > 0) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace

namespace {

// ---- scratch of the allocation-free decode (attn_decode_fwd_noalloc)
//
// The split partials and the partition plan of a decode go to this file-scope device
// array instead of a caller workspace. Each device the library runs on holds its own copy
// until the process ends. In host code the array's name is only a host-side stand-in:
// its device address is looked up once per device, with that device current, and only
// that address is ever passed to kernels.
static __device__ __align__(256) char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`.
attn_status_t scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(ATTN_ERR_NO_DEVICE, "no current HIP device");
  }
  if (dev >= kMaxDevices) return fail(ATTN_ERR_UNSUPPORTED, "device index %d above %d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(ATTN_ERR_LAUNCH, "hipGetSymbolAddress of the decode scratch failed on device %d: %s", dev,
                  hipGetErrorString(e));
    }
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return ATTN_OK;
}

// The decode of attn_decode_fwd and attn_decode_fwd_noalloc: the caller's workspace, or
// (noalloc) this device's copy of the static scratch array.
attn_status_t decode_impl(const attn_decode_args_t* a, void* stream, bool noalloc) {
  const char* fn = noalloc ? "attn_decode_fwd_noalloc" : "attn_decode_fwd";
  try {
    if (!a) return fail(ATTN_ERR_INVALID_ARG, "args is NULL");
    if (a->batch < 0) return fail(ATTN_ERR_INVALID_ARG, "batch must be >= 0");
    if (a->qkv_dtype != ATTN_F16 && a->qkv_dtype != ATTN_BF16)
      return fail(ATTN_ERR_INVALID_ARG, "qkv_dtype must be ATTN_F16 or ATTN_BF16");
    if (a->o_dtype != ATTN_F16 && a->o_dtype != ATTN_BF16 && a->o_dtype != ATTN_F32)
      return fail(ATTN_ERR_INVALID_ARG, "o_dtype must be ATTN_F16, ATTN_BF16 or ATTN_F32");
    if (attn_status_t st = check_round(a->o_round, a->o_dtype); st != ATTN_OK) return st;
    if (!valid_d(a->head_dim)) return fail(ATTN_ERR_INVALID_ARG, "head_dim must be 64, 128 or 256 (got %d)", a->head_dim);
    if (a->num_heads_q <= 0 || a->num_heads_kv <= 0)
      return fail(ATTN_ERR_INVALID_ARG, "head counts must be positive");
    if (a->num_heads_q % a->num_heads_kv != 0)
      return fail(ATTN_ERR_INVALID_ARG, "num_heads_q (%d) must be a multiple of num_heads_kv (%d)",
                  a->num_heads_q, a->num_heads_kv);
    const int G = a->num_heads_q / a->num_heads_kv;
    if (G > 16) return fail(ATTN_ERR_UNSUPPORTED, "decode supports GQA ratios up to 16 (got %d)", G);
    if (a->num_splits < 1 || a->num_splits > ATTN_MAX_SPLITS)
      return fail(ATTN_ERR_INVALID_ARG, "num_splits must be in [1, %d]", ATTN_MAX_SPLITS);
    if (a->max_seqlen_k < 0) return fail(ATTN_ERR_INVALID_ARG, "max_seqlen_k must be >= 0");
    if (a->max_seqlen_k > ATTN_MAX_SEQLEN)
      return fail(ATTN_ERR_UNSUPPORTED, "max_seqlen_k must be <= %d (got %d)", ATTN_MAX_SEQLEN, a->max_seqlen_k);
    if (a->num_blocks <= 0 || a->max_blocks_per_seq <= 0)
      return fail(ATTN_ERR_INVALID_ARG, "num_blocks and max_blocks_per_seq must be positive");
    if ((int64_t)a->max_blocks_per_seq * ATTN_PAGE_SIZE < a->max_seqlen_k)
      return fail(ATTN_ERR_INVALID_ARG, "block table holds %lld keys, fewer than max_seqlen_k = %d",
                  (long long)a->max_blocks_per_seq * ATTN_PAGE_SIZE, a->max_seqlen_k);
    if (!(std::isfinite(a->scale) && a->scale >= 0.f)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite and >= 0");
    if (a->batch > kMaxGridYZ || a->num_heads_kv > kMaxGridYZ)
      return fail(ATTN_ERR_UNSUPPORTED, "batch and num_heads_kv must be <= %lld", (long long)kMaxGridYZ);
    if (a->batch == 0) return ok();
    if (!a->q || !a->k_cache || !a->v_cache || !a->o || !a->block_table || !a->seqlens_k)
      return fail(ATTN_ERR_INVALID_ARG, "q, k_cache, v_cache, block_table, seqlens_k, o%s must be non-NULL",
                  noalloc ? "" : " and workspace");
    if (!noalloc && !a->workspace)
      return fail(ATTN_ERR_INVALID_ARG, "q, k_cache, v_cache, block_table, seqlens_k, o and workspace must be non-NULL");
    if (!aligned16(a->q) || !aligned16(a->k_cache) || !aligned16(a->v_cache) || !aligned4(a->o))
      return fail(ATTN_ERR_INVALID_ARG, "q, k_cache and v_cache must be 16-byte aligned, o 4-byte aligned");
    if (!aligned4(a->block_table) || !aligned4(a->seqlens_k) || (a->lse && !aligned4(a->lse)))
      return fail(ATTN_ERR_INVALID_ARG, "block_table, seqlens_k and lse must be 4-byte aligned");
    const size_t need = attn_decode_workspace_bytes(a->batch, a->num_heads_q, a->num_splits, a->head_dim);
    if (noalloc) {
      if (a->workspace || a->workspace_bytes)
        return fail(ATTN_ERR_INVALID_ARG, "attn_decode_fwd_noalloc takes no workspace (pass NULL and 0 bytes)");
      if (need > ATTN_NOALLOC_SCRATCH_BYTES)
        return fail(ATTN_ERR_INVALID_ARG,
                    "this decode needs %zu bytes of scratch, above the %zu-byte maximum of "
                    "attn_decode_fwd_noalloc (use attn_decode_fwd with a workspace)",
                    need, (size_t)ATTN_NOALLOC_SCRATCH_BYTES);
    } else {
      if ((reinterpret_cast<uintptr_t>(a->workspace) & 255u) != 0)
        return fail(ATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
      if (a->workspace_bytes < need)
        return fail(ATTN_ERR_INVALID_ARG, "workspace has %zu bytes, needs %zu", a->workspace_bytes, need);
    }

    if (attn_status_t st = device_ready(); st != ATTN_OK) return st;
    void* wsp = a->workspace;
    if (noalloc) {
      if (attn_status_t st = scratch_address(&wsp); st != ATTN_OK) return st;
    }
    const int64_t rows = (int64_t)a->batch * a->num_heads_q * a->num_splits;
    char* ws = static_cast<char*>(wsp);
    float* part_o = reinterpret_cast<float*>(ws);
    const size_t lse_off = align256((size_t)rows * a->head_dim * sizeof(float));
    float* part_lse = reinterpret_cast<float*>(ws + lse_off);
    const size_t plan_off = lse_off + align256((size_t)rows * sizeof(float));
    int32_t* plan = reinterpret_cast<int32_t*>(ws + plan_off);
    int32_t* prefix = reinterpret_cast<int32_t*>(ws + plan_off + 256);
    int32_t* start = reinterpret_cast<int32_t*>(ws + plan_off + 256 +
                                                align256((size_t)(a->batch + 1) * sizeof(int32_t)));
    int part = (a->max_seqlen_k + a->num_splits - 1) / a->num_splits;
    part = ((part + ATTN_PAGE_SIZE - 1) / ATTN_PAGE_SIZE) * ATTN_PAGE_SIZE;
    if (part == 0) part = ATTN_PAGE_SIZE;

    attn::DecodeParams p{};
    p.q = static_cast<const uint16_t*>(a->q);
    p.k = static_cast<const uint16_t*>(a->k_cache);
    p.v = static_cast<const uint16_t*>(a->v_cache);
    p.block_table = a->block_table; p.seqlens_k = a->seqlens_k;
    p.part_o = part_o; p.part_lse = part_lse;
    p.batch = a->batch; p.hq = a->num_heads_q; p.hkv = a->num_heads_kv; p.group = G;
    p.num_blocks = a->num_blocks; p.max_blocks = a->max_blocks_per_seq;
    p.max_seqlen_k = a->max_seqlen_k; p.num_splits = a->num_splits; p.part_tokens = part;
    const float scale = a->scale > 0.f ? a->scale : 1.0f / std::sqrt((float)a->head_dim);
    p.scale_log2 = scale * 1.4426950408889634f;

    p.plan = plan; p.prefix = prefix; p.start = start;

    attn::CombineParams c{};
    c.part_o = part_o; c.part_lse = part_lse; c.o = a->o; c.lse = a->lse;
    c.pairs = a->batch * a->num_heads_q; c.num_splits = a->num_splits; c.o_dtype = a->o_dtype;
    c.o_round = a->o_dtype == ATTN_BF16 ? a->o_round : 0;

    const hipStream_t s = static_cast<hipStream_t>(stream);
    // Balanced split kernel when partitions may be cut (num_splits >= 2) and the page
    // count per KV head fits in int32; otherwise one workgroup per fixed partition.
    const int64_t rmax = ((int64_t)a->max_seqlen_k + ATTN_PAGE_SIZE - 1) / ATTN_PAGE_SIZE;
    const int cus = device_cus();
    if (a->num_splits >= 2 && (int64_t)a->batch * rmax < (int64_t(1) << 30) && cus > 0) {
      // persistent workgroups per KV head: two per CU at d <= 128 (their rings take half
      // the LDS each), one at d = 256
      const int per_cu = a->head_dim <= 128 ? 2 : 1;
      p.nwk = std::max(1, std::min(kMaxStreamWG, per_cu * cus / a->num_heads_kv));
      c.seqlens_k = a->seqlens_k; c.heads = a->num_heads_q; c.max_seqlen_k = a->max_seqlen_k;
      if (attn_status_t st = launch_status(attn::launch_decode_stream(p, a->head_dim, a->qkv_dtype, s),
                                           "decode split");
          st != ATTN_OK)
        return st;
    } else if (attn_status_t st = launch_status(attn::launch_decode_split(p, a->head_dim, a->qkv_dtype, s),
                                                "decode split");
               st != ATTN_OK) {
      return st;
    }
    return launch_status(attn::launch_combine(c, a->head_dim, s), "decode combine");
  } catch (...) {
    return fail(ATTN_ERR_LAUNCH, "internal error in %s", fn);
  }
}


}  // namespace

extern "C" {

int32_t attn_abi_version(void) { return ATTN_ABI_VERSION; }

const char* attn_last_error(void) { return g_last_error.c_str(); }

int32_t attn_device_count(void) {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

attn_status_t attn_device_info(int32_t device, attn_device_info_t* info) {
  try {
    if (!info) return fail(ATTN_ERR_INVALID_ARG, "info is NULL");
    if (device < 0) return fail(ATTN_ERR_INVALID_ARG, "device must be >= 0 (got %d)", device);
    if (attn_status_t st = device_ready(); st != ATTN_OK) return st;
    const int n = attn_device_count();
    if (device >= n) return fail(ATTN_ERR_INVALID_ARG, "device %d is not visible (%d device(s))", device, n);
    hipDeviceProp_t prop{};
    if (hipError_t e = hipGetDeviceProperties(&prop, device); e != hipSuccess)
      return fail(ATTN_ERR_LAUNCH, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
    *info = attn_device_info_t{};
    snprintf(info->name, sizeof(info->name), "%s", prop.name);
    snprintf(info->arch, sizeof(info->arch), "%s", prop.gcnArchName);
    info->total_memory = (int64_t)prop.totalGlobalMem;
    info->compute_units = prop.multiProcessorCount;
    info->clock_khz = prop.clockRate;
    info->memory_clock_khz = prop.memoryClockRate;
    info->memory_bus_bits = prop.memoryBusWidth;
    info->lds_per_cu = (int32_t)prop.maxSharedMemoryPerMultiProcessor;
    info->l2_bytes = prop.l2CacheSize;
    int rv = 0, dv = 0;
    if (hipRuntimeGetVersion(&rv) != hipSuccess) rv = 0;
    if (hipDriverGetVersion(&dv) != hipSuccess) dv = 0;
    info->runtime_version = rv;
    info->driver_version = dv;
    return ok();
  } catch (...) {
    return fail(ATTN_ERR_LAUNCH, "internal error in attn_device_info");
  }
}

}  // extern "C"

namespace {

// Host-side checks of a prefill call's sizes, enums and alignments (pointers are not
// required to be set) and its kernel parameters.
attn_status_t prefill_setup(const attn_prefill_args_t* a, attn::PrefillParams* p) {
  if (!a) return fail(ATTN_ERR_INVALID_ARG, "args is NULL");
  if (a->batch < 0 || a->seqlen_q < 0) return fail(ATTN_ERR_INVALID_ARG, "batch and seqlen_q must be >= 0");
  if (a->qkv_dtype != ATTN_F16 && a->qkv_dtype != ATTN_BF16)
    return fail(ATTN_ERR_INVALID_ARG, "qkv_dtype must be ATTN_F16 or ATTN_BF16");
  if (a->o_dtype != ATTN_F16 && a->o_dtype != ATTN_BF16 && a->o_dtype != ATTN_F32)
    return fail(ATTN_ERR_INVALID_ARG, "o_dtype must be ATTN_F16, ATTN_BF16 or ATTN_F32");
  if (attn_status_t st = check_round(a->o_round, a->o_dtype); st != ATTN_OK) return st;
  if (a->layout != ATTN_BSHD && a->layout != ATTN_BHSD)
    return fail(ATTN_ERR_INVALID_ARG, "layout must be ATTN_BSHD or ATTN_BHSD");
  if (a->causal != 0 && a->causal != 1) return fail(ATTN_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (a->precise != 0 && a->precise != 1) return fail(ATTN_ERR_INVALID_ARG, "precise must be 0 or 1");
  if (!valid_d(a->head_dim)) return fail(ATTN_ERR_INVALID_ARG, "head_dim must be 64, 128 or 256 (got %d)", a->head_dim);
  if (a->num_heads_q <= 0 || a->num_heads_kv <= 0)
    return fail(ATTN_ERR_INVALID_ARG, "head counts must be positive");
  if (a->num_heads_q % a->num_heads_kv != 0)
    return fail(ATTN_ERR_INVALID_ARG, "num_heads_q (%d) must be a multiple of num_heads_kv (%d)",
                a->num_heads_q, a->num_heads_kv);
  const int G = a->num_heads_q / a->num_heads_kv;
  if (G > 128) return fail(ATTN_ERR_UNSUPPORTED, "GQA ratio %d above 128 is not supported", G);
  if (a->seqlen_k < 0) return fail(ATTN_ERR_INVALID_ARG, "seqlen_k must be >= 0");
  if (a->seqlen_q > ATTN_MAX_SEQLEN || a->seqlen_k > ATTN_MAX_SEQLEN)
    return fail(ATTN_ERR_UNSUPPORTED, "seqlen_q and seqlen_k must be <= %d", ATTN_MAX_SEQLEN);
  if (!(std::isfinite(a->scale) && a->scale >= 0.f)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite and >= 0");
  if (a->batch > kMaxGridYZ || a->num_heads_kv > kMaxGridYZ)
    return fail(ATTN_ERR_UNSUPPORTED, "batch and num_heads_kv must be <= %lld", (long long)kMaxGridYZ);
  const bool paged = a->block_table != nullptr;
  if (paged) {
    if (!a->seqlens_k) return fail(ATTN_ERR_INVALID_ARG, "paged K/V requires seqlens_k");
    if (a->num_blocks <= 0 || a->max_blocks_per_seq <= 0)
      return fail(ATTN_ERR_INVALID_ARG, "paged K/V requires num_blocks > 0 and max_blocks_per_seq > 0");
    if ((int64_t)a->max_blocks_per_seq * ATTN_PAGE_SIZE < a->seqlen_k)
      return fail(ATTN_ERR_INVALID_ARG, "block table holds %lld keys, fewer than seqlen_k = %d",
                  (long long)a->max_blocks_per_seq * ATTN_PAGE_SIZE, a->seqlen_k);
    if (!aligned4(a->block_table)) return fail(ATTN_ERR_INVALID_ARG, "block_table must be 4-byte aligned");
  }
  if (a->seqlens_k && !aligned4(a->seqlens_k)) return fail(ATTN_ERR_INVALID_ARG, "seqlens_k must be 4-byte aligned");
  if (a->cu_seqlens_q) {
    if (a->layout != ATTN_BSHD) return fail(ATTN_ERR_INVALID_ARG, "packed queries (cu_seqlens_q) need the BSHD layout");
    if (!aligned4(a->cu_seqlens_q)) return fail(ATTN_ERR_INVALID_ARG, "cu_seqlens_q must be 4-byte aligned");
  }
  if (a->kv_splits < 0 || a->kv_splits > ATTN_MAX_SPLITS)
    return fail(ATTN_ERR_INVALID_ARG, "kv_splits must be in [0, %d] (got %d)", ATTN_MAX_SPLITS, a->kv_splits);
  const int64_t D = a->head_dim, Sq = a->seqlen_q, Sk = a->seqlen_k;
  const int64_t Hq = a->num_heads_q, Hkv = a->num_heads_kv;
  p->q = static_cast<const uint16_t*>(a->q);
  p->k = static_cast<const uint16_t*>(a->k);
  p->v = static_cast<const uint16_t*>(a->v);
  p->o = a->o;
  p->lse = a->lse;
  p->block_table = a->block_table;
  p->seqlens_k = a->seqlens_k;
  if (a->layout == ATTN_BSHD) {
    p->q_sb = Sq * Hq * D; p->q_sh = D; p->q_ss = Hq * D;
    p->kv_sb = Sk * Hkv * D; p->kv_sh = D; p->kv_ss = Hkv * D;
  } else {
    p->q_sb = Hq * Sq * D; p->q_sh = Sq * D; p->q_ss = D;
    p->kv_sb = Hkv * Sk * D; p->kv_sh = Sk * D; p->kv_ss = D;
  }
  if (a->cu_seqlens_q) p->q_sb = 0;   // packed: rows of every sequence in one [total_q, Hq, d]
  p->o_sb = p->q_sb; p->o_sh = p->q_sh; p->o_ss = p->q_ss;
  p->cu_seqlens_q = a->cu_seqlens_q;
  p->batch = a->batch; p->hq = a->num_heads_q; p->hkv = a->num_heads_kv; p->group = G;
  p->seqlen_q = a->seqlen_q; p->seqlen_k = a->seqlen_k;
  p->num_blocks = a->num_blocks; p->max_blocks = a->max_blocks_per_seq;
  p->bq = 128 / G;
  p->causal = a->causal; p->o_dtype = a->o_dtype;
  p->o_round = a->o_dtype == ATTN_BF16 ? a->o_round : 0;
  const float scale = a->scale > 0.f ? a->scale : 1.0f / std::sqrt((float)a->head_dim);
  p->scale_log2 = scale * 1.4426950408889634f;
  return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status_t attn_prefill_fwd(const attn_prefill_args_t* a, void* stream) {
  try {
    attn::PrefillParams p{};
    if (attn_status_t st = prefill_setup(a, &p); st != ATTN_OK) return st;
    if (a->workspace && (reinterpret_cast<uintptr_t>(a->workspace) & 255u) != 0)
      return fail(ATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    if (!a->workspace && a->workspace_bytes != 0)
      return fail(ATTN_ERR_INVALID_ARG, "workspace_bytes must be 0 without a workspace");
    if (a->kv_splits >= 2 && !a->workspace)
      return fail(ATTN_ERR_INVALID_ARG, "kv_splits = %d needs a workspace (attn_prefill_workspace_bytes)", a->kv_splits);
    if (a->batch == 0 || a->seqlen_q == 0) return ok();
    if (!a->q || !a->k || !a->v || !a->o) return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o must be non-NULL");
    if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o))
      return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
    if (a->lse && !aligned4(a->lse)) return fail(ATTN_ERR_INVALID_ARG, "lse must be 4-byte aligned");

    if (attn_status_t st = device_ready(); st != ATTN_OK) return st;
    p.cus = device_cus();
    attn::PrefillPlan plan{};
    if (hipError_t e = attn::plan_prefill(p, a->head_dim, a->qkv_dtype, a->precise != 0,
                                          a->workspace ? a->kv_splits : 1, &plan);
        e != hipSuccess)
      return fail(ATTN_ERR_LAUNCH, "prefill plan failed: %s", hipGetErrorString(e));
    if (plan.parts >= 2) {
      if (a->workspace_bytes < plan.bytes)
        return fail(ATTN_ERR_INVALID_ARG, "workspace of %zu bytes, the tail split needs %zu",
                    a->workspace_bytes, plan.bytes);
      char* ws = static_cast<char*>(a->workspace);
      p.part_o = reinterpret_cast<float*>(ws + plan.part_o_off);
      p.part_lse = reinterpret_cast<float*>(ws + plan.part_lse_off);
      p.row_off = reinterpret_cast<int64_t*>(ws + plan.row_off_off);
      p.row_lse = reinterpret_cast<int64_t*>(ws + plan.row_lse_off);
    }
    return launch_status(attn::launch_prefill(p, plan, a->head_dim, a->qkv_dtype, a->precise != 0,
                                              static_cast<hipStream_t>(stream)),
                         "prefill");
  } catch (...) {
    return fail(ATTN_ERR_LAUNCH, "internal error in attn_prefill_fwd");
  }
}

size_t attn_prefill_workspace_bytes(const attn_prefill_args_t* a) {
  // a size query: the checks below leave the thread's last error message as it was
  const std::string saved = g_last_error;
  struct Restore {
    const std::string& s;
    ~Restore() { g_last_error = s; }
  } restore{saved};
  try {
    attn::PrefillParams p{};
    if (prefill_setup(a, &p) != ATTN_OK) return 0;
    if (a->batch == 0 || a->seqlen_q == 0 || a->kv_splits == 1) return 0;
    if (device_ready() != ATTN_OK) return 0;
    p.cus = device_cus();
    attn::PrefillPlan plan{};
    if (attn::plan_prefill(p, a->head_dim, a->qkv_dtype, a->precise != 0, a->kv_splits, &plan) != hipSuccess) {
      (void)hipGetLastError();
      return 0;
    }
    return plan.parts >= 2 ? plan.bytes : 0;
  } catch (...) {
    return 0;
  }
}

size_t attn_decode_workspace_bytes(int32_t batch, int32_t num_heads_q, int32_t num_splits,
                                   int32_t head_dim) {
  if (batch <= 0 || num_heads_q <= 0 || num_splits <= 0 || num_splits > ATTN_MAX_SPLITS || !valid_d(head_dim))
    return 0;
  const size_t rows = (size_t)batch * num_heads_q * num_splits;
  return align256(rows * head_dim * sizeof(float)) + align256(rows * sizeof(float)) +
         plan_bytes(batch);
}

attn_status_t attn_splitkv_combine(const attn_combine_args_t* a, void* stream) {
  try {
    if (!a) return fail(ATTN_ERR_INVALID_ARG, "args is NULL");
    if (a->batch < 0 || a->num_heads < 0) return fail(ATTN_ERR_INVALID_ARG, "batch and num_heads must be >= 0");
    if (a->num_splits < 1 || a->num_splits > ATTN_MAX_SPLITS)
      return fail(ATTN_ERR_INVALID_ARG, "num_splits must be in [1, %d]", ATTN_MAX_SPLITS);
    if (!valid_d(a->head_dim)) return fail(ATTN_ERR_INVALID_ARG, "head_dim must be 64, 128 or 256");
    if (a->o_dtype != ATTN_F16 && a->o_dtype != ATTN_BF16 && a->o_dtype != ATTN_F32)
      return fail(ATTN_ERR_INVALID_ARG, "o_dtype must be ATTN_F16, ATTN_BF16 or ATTN_F32");
    if (attn_status_t st = check_round(a->o_round, a->o_dtype); st != ATTN_OK) return st;
    const int64_t pairs = (int64_t)a->batch * a->num_heads;
    if (pairs == 0) return ok();
    if (pairs > (int64_t)1 << 30) return fail(ATTN_ERR_UNSUPPORTED, "batch * num_heads too large");
    if (!a->partial_o || !a->partial_lse || !a->o)
      return fail(ATTN_ERR_INVALID_ARG, "partial_o, partial_lse and o must be non-NULL");
    if (!aligned4(a->partial_o) || !aligned4(a->partial_lse) || !aligned4(a->o) || (a->lse && !aligned4(a->lse)))
      return fail(ATTN_ERR_INVALID_ARG, "buffers must be 4-byte aligned");
    attn::CombineParams p{};
    p.part_o = a->partial_o; p.part_lse = a->partial_lse; p.o = a->o; p.lse = a->lse;
    p.pairs = (int32_t)pairs; p.num_splits = a->num_splits; p.o_dtype = a->o_dtype;
    p.o_round = a->o_dtype == ATTN_BF16 ? a->o_round : 0;
    if (attn_status_t st = device_ready(); st != ATTN_OK) return st;
    return launch_status(attn::launch_combine(p, a->head_dim, static_cast<hipStream_t>(stream)), "combine");
  } catch (...) {
    return fail(ATTN_ERR_LAUNCH, "internal error in attn_splitkv_combine");
  }
}

attn_status_t attn_decode_fwd(const attn_decode_args_t* a, void* stream) {
  return decode_impl(a, stream, false);
}

attn_status_t attn_decode_fwd_noalloc(const attn_decode_args_t* a, void* stream) {
  return decode_impl(a, stream, true);
}

}  // extern "C"
