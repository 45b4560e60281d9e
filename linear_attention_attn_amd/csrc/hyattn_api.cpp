// hyattn C ABI: argument validation, the state-slot pool, checked mode,
// kernel dispatch and the per-layer hybrid step. See include/hyattn.h.
//
// Pages: "P2" = "推理框架适配Hybrid Model：KV Cache管理与算子调度实战",
//        "P1" = "Hybrid Model推理适配：vLLM与SGLang的工程实践指南".
#include "hyattn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "hy_kernels.hpp"

static_assert(HYATTN_NOALLOC_SCRATCH_BYTES == hy::kDecodeScratchBytes,
              "the header states the scratch size of the allocation-free decode");

struct hyattn_state_pool {
  float* base;
  size_t bytes;
  int n_layers, n_slots, H, D;
  std::vector<unsigned char> used;    // slot allocated
  std::vector<unsigned char> zeroed;  // slot zeroed since its allocation
  std::mutex mu;
};

namespace {

thread_local std::string g_err;

hyattn_status fail(hyattn_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

hyattn_status ok() {
  g_err.clear();
  return HYATTN_OK;
}

bool checked_mode() {
  const char* e = getenv("HYATTN_CHECK");
  return e && e[0] && strcmp(e, "0") != 0;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// A second stream per device (default priority) and the two events that fork
// work onto it from the caller's stream and join it back. The hybrid step
// runs a full layer's decode attention there beside the layer's prefill
// attention: they read disjoint requests of the pools, and a decode
// workgroup fits a CU beside a prefill workgroup (the prefill's matrix work
// and the decode's HBM streaming then overlap). Created on first use, kept
// until the process ends. Callers hold `mu` from fork to join, so steps
// launched from several host threads onto one device take turns at that
// point.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  std::mutex mu;
};

hipError_t side_stream(SideStream** out) {
  static std::mutex mu;
  static SideStream per_dev[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  SideStream& ss = per_dev[dev];
  if (!ss.s) {
    hipStream_t st = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    if ((e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&f, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&j, hipEventDisableTiming)) != hipSuccess) {
      if (f) hipEventDestroy(f);
      hipStreamDestroy(st);
      return e;
    }
    ss.s = st;
    ss.fork = f;
    ss.join = j;
  }
  *out = &ss;
  return hipSuccess;
}

hyattn_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(HYATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool dtype_ok(hyattn_dtype dt) { return dt == HYATTN_F32 || dt == HYATTN_BF16; }
bool d_ok(int D) { return D == 64 || D == 128; }

// Copy a device array to the host, synchronously on `s` (checked mode).
template <typename T>
hyattn_status fetch(std::vector<T>& out, const T* dev, size_t n, hipStream_t s) {
  out.resize(n);
  if (n == 0) return ok();
  hipError_t e = hipMemcpyAsync(out.data(), dev, n * sizeof(T), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return hip_status(e, "checked mode: reading an argument array");
}

hyattn_status check_slots(hyattn_state_pool* p, const int32_t* slots_dev, int n, hipStream_t s,
                          bool need_zeroed) {
  std::vector<int32_t> h;
  hyattn_status st = fetch(h, slots_dev, (size_t)n, s);
  if (st != HYATTN_OK) return st;
  std::lock_guard<std::mutex> lk(p->mu);
  std::vector<unsigned char> seen(p->n_slots, 0);
  for (int i = 0; i < n; ++i) {
    const int id = h[i];
    if (id < 0 || id >= p->n_slots)
      return fail(HYATTN_ERR_BAD_SLOT, "slot %d (entry %d) outside [0, %d)", id, i, p->n_slots);
    if (!p->used[id]) return fail(HYATTN_ERR_BAD_SLOT, "slot %d (entry %d) is not allocated", id, i);
    if (need_zeroed && !p->zeroed[id])
      return fail(HYATTN_ERR_BAD_SLOT, "slot %d (entry %d) was never zeroed since allocation", id, i);
    if (seen[id]) return fail(HYATTN_ERR_INVALID_ARG, "slot %d appears twice in one call", id);
    seen[id] = 1;
  }
  return ok();
}

// Checked-mode validation of cumulative lengths: cu[0] == 0, non-decreasing,
// every length <= max_len, total <= max_total (if >= 0).
hyattn_status check_cu(const std::vector<int32_t>& cu, int max_len, const char* name) {
  if (cu.empty() || cu[0] != 0) return fail(HYATTN_ERR_INVALID_ARG, "%s[0] must be 0", name);
  for (size_t i = 1; i < cu.size(); ++i) {
    const int len = cu[i] - cu[i - 1];
    if (len < 0) return fail(HYATTN_ERR_INVALID_ARG, "%s decreases at %zu", name, i);
    if (max_len >= 0 && len > max_len)
      return fail(HYATTN_ERR_INVALID_ARG, "%s: length %d at %zu exceeds bound %d", name, len, i - 1,
                  max_len);
  }
  return ok();
}

// Checked-mode validation of block tables against context lengths.
hyattn_status check_tables(const int32_t* bt_dev, int B, int max_blocks, const int32_t* ctx_dev,
                           int max_context, int64_t n_blocks, hipStream_t s,
                           std::vector<int32_t>* ctx_out = nullptr) {
  std::vector<int32_t> bt, ctx;
  hyattn_status st = fetch(ctx, ctx_dev, (size_t)B, s);
  if (st != HYATTN_OK) return st;
  st = fetch(bt, bt_dev, (size_t)B * max_blocks, s);
  if (st != HYATTN_OK) return st;
  for (int r = 0; r < B; ++r) {
    const int c = ctx[r];
    if (c < 0 || c > max_context)
      return fail(HYATTN_ERR_INVALID_ARG, "context_lens[%d] = %d outside [0, %d]", r, c, max_context);
    const int nb = (c + 15) / 16;
    if (nb > max_blocks)
      return fail(HYATTN_ERR_INVALID_ARG, "context_lens[%d] = %d needs %d blocks > %d", r, c, nb,
                  max_blocks);
    for (int j = 0; j < nb; ++j) {
      const int32_t b = bt[(size_t)r * max_blocks + j];
      if (b < 0 || b >= n_blocks)
        return fail(HYATTN_ERR_INVALID_ARG, "block_tables[%d][%d] = %d outside [0, %lld)", r, j, b,
                    (long long)n_blocks);
    }
  }
  if (ctx_out) *ctx_out = ctx;
  return ok();
}

hyattn_status check_pool_layer(const hyattn_state_pool* p, int layer) {
  if (!p) return fail(HYATTN_ERR_INVALID_ARG, "state pool is NULL");
  if (layer < 0 || layer >= p->n_layers)
    return fail(HYATTN_ERR_INVALID_ARG, "linear layer %d outside [0, %d)", layer, p->n_layers);
  return ok();
}

float* layer_base(const hyattn_state_pool* p, int layer) {
  return p->base + (size_t)layer * p->n_slots * p->H * (size_t)p->D * p->D;
}

bool prefill_chunk_ok(int D, int chunk, hyattn_dtype dt, bool gated) {
  if (dt == HYATTN_F32) return chunk >= 1 && chunk <= hy::kMaxChunkF32;
  if (chunk < 16 || chunk > 256 || chunk % 16 != 0) return false;
  return hy::linear_prefill_bf16_lds_bytes(D, chunk, gated) <= 160 * 1024;
}

// Checked mode: the gated variant's log forget factors are finite and <= 0.
hyattn_status check_log_gamma(const float* g_dev, size_t n, hipStream_t s) {
  std::vector<float> g;
  hyattn_status st = fetch(g, g_dev, n, s);
  if (st != HYATTN_OK) return st;
  for (size_t i = 0; i < n; ++i)
    if (!(g[i] <= 0.f) || !std::isfinite(g[i]))
      return fail(HYATTN_ERR_INVALID_ARG, "log_gamma[%zu] = %g is not a finite value <= 0", i,
                  (double)g[i]);
  return HYATTN_OK;
}

}  // namespace

extern "C" {

const char* hyattn_last_error(void) { return g_err.c_str(); }

int hyattn_abi_version(void) { return 2; }

// ---------------------------------------------------------------- state pool --
size_t hyattn_state_pool_bytes(int n_linear_layers, int n_slots, int H, int D) {
  if (n_linear_layers < 0 || n_slots < 0 || H < 0 || D < 0) return 0;
  const unsigned __int128 b = (unsigned __int128)n_linear_layers * (unsigned)n_slots * (unsigned)H *
                              (unsigned)D * (unsigned)D * 4u;
  if (b > (unsigned __int128)SIZE_MAX) return 0;
  return (size_t)b;
}

hyattn_status hyattn_state_pool_create(void* dev_buf, size_t bytes, int n_linear_layers,
                                       int n_slots, int H, int D, hyattn_state_pool** out) {
  if (!out) return fail(HYATTN_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (n_linear_layers < 1 || n_slots < 1 || H < 1)
    return fail(HYATTN_ERR_INVALID_ARG, "pool dims must be positive (L=%d, slots=%d, H=%d)",
                n_linear_layers, n_slots, H);
  if (!d_ok(D)) return fail(HYATTN_ERR_UNSUPPORTED, "head dim %d not supported (64 or 128)", D);
  if ((int64_t)H * D >= (1 << 23))
    return fail(HYATTN_ERR_UNSUPPORTED, "H * D = %lld not supported (at most 2^23 - 1)",
                (long long)H * D);
  const size_t need = hyattn_state_pool_bytes(n_linear_layers, n_slots, H, D);
  if (need == 0) return fail(HYATTN_ERR_INVALID_ARG, "pool size overflows");
  if (!dev_buf) return fail(HYATTN_ERR_INVALID_ARG, "device buffer is NULL");
  if (reinterpret_cast<uintptr_t>(dev_buf) % 16)
    return fail(HYATTN_ERR_INVALID_ARG, "device buffer must be 16-byte aligned");
  if (bytes < need)
    return fail(HYATTN_ERR_INVALID_ARG, "buffer has %zu bytes, pool needs %zu", bytes, need);
  hyattn_state_pool* p = new (std::nothrow) hyattn_state_pool();
  if (!p) return fail(HYATTN_ERR_INVALID_ARG, "host allocation failed");
  p->base = static_cast<float*>(dev_buf);
  p->bytes = bytes;
  p->n_layers = n_linear_layers;
  p->n_slots = n_slots;
  p->H = H;
  p->D = D;
  p->used.assign(n_slots, 0);
  p->zeroed.assign(n_slots, 0);
  *out = p;
  return ok();
}

hyattn_status hyattn_state_pool_destroy(hyattn_state_pool* pool) {
  delete pool;
  return ok();
}

hyattn_status hyattn_state_pool_alloc(hyattn_state_pool* p, int n, int32_t* slots_out) {
  if (!p) return fail(HYATTN_ERR_INVALID_ARG, "state pool is NULL");
  if (n < 0) return fail(HYATTN_ERR_INVALID_ARG, "n = %d < 0", n);
  if (n > 0 && !slots_out) return fail(HYATTN_ERR_INVALID_ARG, "slots_out is NULL");
  std::lock_guard<std::mutex> lk(p->mu);
  int free_n = 0;
  for (int i = 0; i < p->n_slots; ++i) free_n += !p->used[i];
  if (free_n < n)
    return fail(HYATTN_ERR_OUT_OF_SLOTS, "state pool exhausted: %d requested, %d of %d free", n,
                free_n, p->n_slots);
  int k = 0;
  for (int i = 0; i < p->n_slots && k < n; ++i)
    if (!p->used[i]) {
      p->used[i] = 1;
      p->zeroed[i] = 0;
      slots_out[k++] = i;
    }
  return ok();
}

hyattn_status hyattn_state_pool_zero(hyattn_state_pool* p, const int32_t* slots_dev, int n,
                                     void* stream) {
  if (!p) return fail(HYATTN_ERR_INVALID_ARG, "state pool is NULL");
  if (n < 0) return fail(HYATTN_ERR_INVALID_ARG, "n = %d < 0", n);
  if (n == 0) return ok();
  if (!slots_dev) return fail(HYATTN_ERR_INVALID_ARG, "slots is NULL");
  hipStream_t s = as_stream(stream);
  std::vector<int32_t> h;
  if (checked_mode()) {
    hyattn_status st = check_slots(p, slots_dev, n, s, false);
    if (st != HYATTN_OK) return st;
    fetch(h, slots_dev, (size_t)n, s);
  }
  hipError_t e = hy::launch_state_zero(p->base, p->n_layers, p->n_slots,
                                       (int64_t)p->H * p->D * p->D, slots_dev, n, s);
  if (e != hipSuccess) return hip_status(e, "state zero launch");
  if (!h.empty()) {
    std::lock_guard<std::mutex> lk(p->mu);
    for (int id : h) p->zeroed[id] = 1;
  }
  return ok();
}

hyattn_status hyattn_state_pool_free(hyattn_state_pool* p, const int32_t* slots, int n) {
  if (!p) return fail(HYATTN_ERR_INVALID_ARG, "state pool is NULL");
  if (n < 0) return fail(HYATTN_ERR_INVALID_ARG, "n = %d < 0", n);
  if (n > 0 && !slots) return fail(HYATTN_ERR_INVALID_ARG, "slots is NULL");
  std::lock_guard<std::mutex> lk(p->mu);
  std::vector<unsigned char> seen(p->n_slots, 0);
  for (int i = 0; i < n; ++i) {
    const int id = slots[i];
    if (id < 0 || id >= p->n_slots)
      return fail(HYATTN_ERR_BAD_SLOT, "free: slot %d outside [0, %d)", id, p->n_slots);
    if (!p->used[id]) return fail(HYATTN_ERR_BAD_SLOT, "free: slot %d is not allocated", id);
    if (seen[id]) return fail(HYATTN_ERR_BAD_SLOT, "free: slot %d listed twice", id);
    seen[id] = 1;
  }
  for (int i = 0; i < n; ++i) {
    p->used[slots[i]] = 0;
    p->zeroed[slots[i]] = 0;
  }
  return ok();
}

int hyattn_state_pool_in_use(const hyattn_state_pool* p) {
  if (!p) return -1;
  hyattn_state_pool* mp = const_cast<hyattn_state_pool*>(p);
  std::lock_guard<std::mutex> lk(mp->mu);
  int n = 0;
  for (unsigned char u : p->used) n += u;
  return n;
}

void* hyattn_state_pool_state_ptr(const hyattn_state_pool* p, int layer, int slot) {
  if (!p || layer < 0 || layer >= p->n_layers || slot < 0 || slot >= p->n_slots) return nullptr;
  return layer_base(p, layer) + (size_t)slot * p->H * p->D * p->D;
}

// ------------------------------------------------------------- linear layers --
static hyattn_status linear_prefill(hyattn_state_pool* p, int layer, const void* q,
                                    const void* k, const void* v, const float* log_gamma,
                                    void* o, const int32_t* cu_seqlens_dev,
                                    const int32_t* slots_dev, int n_req, int chunk_size,
                                    hyattn_dtype dtype, void* stream, bool gated) {
  hyattn_status st = check_pool_layer(p, layer);
  if (st != HYATTN_OK) return st;
  if (!dtype_ok(dtype)) return fail(HYATTN_ERR_UNSUPPORTED, "dtype %d not supported", (int)dtype);
  if (n_req < 0) return fail(HYATTN_ERR_INVALID_ARG, "n_req = %d < 0", n_req);
  if (!prefill_chunk_ok(p->D, chunk_size, dtype, gated))
    return fail(HYATTN_ERR_UNSUPPORTED,
                "chunk_size %d not supported (bf16: multiple of 16 in [16, 256] that fits LDS; "
                "fp32: [1, %d])",
                chunk_size, hy::kMaxChunkF32);
  if (n_req == 0) return ok();
  if (!q || !k || !v || !o || !cu_seqlens_dev || !slots_dev || (gated && !log_gamma))
    return fail(HYATTN_ERR_INVALID_ARG, "a tensor pointer is NULL");
  hipStream_t s = as_stream(stream);
  if (checked_mode()) {
    std::vector<int32_t> cu;
    if ((st = fetch(cu, cu_seqlens_dev, (size_t)n_req + 1, s)) != HYATTN_OK) return st;
    if ((st = check_cu(cu, -1, "cu_seqlens")) != HYATTN_OK) return st;
    if ((st = check_slots(p, slots_dev, n_req, s, true)) != HYATTN_OK) return st;
    if (gated && (st = check_log_gamma(log_gamma, (size_t)cu[n_req] * p->H, s)) != HYATTN_OK)
      return st;
  }
  return hip_status(hy::launch_linear_prefill(layer_base(p, layer), p->n_slots, q, k, v, o,
                                              gated ? log_gamma : nullptr, cu_seqlens_dev,
                                              slots_dev, n_req, p->H, p->D, chunk_size,
                                              dtype == HYATTN_BF16, s),
                    "linear prefill launch");
}

static hyattn_status linear_decode(hyattn_state_pool* p, int layer, const void* q, const void* k,
                                   const void* v, const float* log_gamma, void* o,
                                   const int32_t* slots_dev, int B, hyattn_dtype dtype,
                                   void* stream, bool gated) {
  hyattn_status st = check_pool_layer(p, layer);
  if (st != HYATTN_OK) return st;
  if (!dtype_ok(dtype)) return fail(HYATTN_ERR_UNSUPPORTED, "dtype %d not supported", (int)dtype);
  if (B < 0) return fail(HYATTN_ERR_INVALID_ARG, "B = %d < 0", B);
  if (B == 0) return ok();
  if (!q || !k || !v || !o || !slots_dev || (gated && !log_gamma))
    return fail(HYATTN_ERR_INVALID_ARG, "a tensor pointer is NULL");
  hipStream_t s = as_stream(stream);
  if (checked_mode()) {
    if ((st = check_slots(p, slots_dev, B, s, true)) != HYATTN_OK) return st;
    if (gated && (st = check_log_gamma(log_gamma, (size_t)B * p->H, s)) != HYATTN_OK) return st;
  }
  return hip_status(hy::launch_linear_decode(layer_base(p, layer), p->n_slots, q, k, v, o,
                                             gated ? log_gamma : nullptr, slots_dev, B, p->H,
                                             p->D, dtype == HYATTN_BF16, s),
                    "linear decode launch");
}

hyattn_status hyattn_linear_prefill_chunked(hyattn_state_pool* p, int layer, const void* q,
                                            const void* k, const void* v, void* o,
                                            const int32_t* cu_seqlens_dev,
                                            const int32_t* slots_dev, int n_req, int chunk_size,
                                            hyattn_dtype dtype, void* stream) {
  return linear_prefill(p, layer, q, k, v, nullptr, o, cu_seqlens_dev, slots_dev, n_req,
                        chunk_size, dtype, stream, false);
}

hyattn_status hyattn_linear_decode(hyattn_state_pool* p, int layer, const void* q, const void* k,
                                   const void* v, void* o, const int32_t* slots_dev, int B,
                                   hyattn_dtype dtype, void* stream) {
  return linear_decode(p, layer, q, k, v, nullptr, o, slots_dev, B, dtype, stream, false);
}

hyattn_status hyattn_linear_prefill_chunked_gated(hyattn_state_pool* p, int layer, const void* q,
                                                  const void* k, const void* v,
                                                  const float* log_gamma, void* o,
                                                  const int32_t* cu_seqlens_dev,
                                                  const int32_t* slots_dev, int n_req,
                                                  int chunk_size, hyattn_dtype dtype,
                                                  void* stream) {
  return linear_prefill(p, layer, q, k, v, log_gamma, o, cu_seqlens_dev, slots_dev, n_req,
                        chunk_size, dtype, stream, true);
}

hyattn_status hyattn_linear_decode_gated(hyattn_state_pool* p, int layer, const void* q,
                                         const void* k, const void* v, const float* log_gamma,
                                         void* o, const int32_t* slots_dev, int B,
                                         hyattn_dtype dtype, void* stream) {
  return linear_decode(p, layer, q, k, v, log_gamma, o, slots_dev, B, dtype, stream, true);
}

// --------------------------------------------------------------- full layers --
static hyattn_status check_full_dims(int B, int H_q, int H_kv, int D, hyattn_dtype dtype,
                                     int64_t n_blocks, int max_blocks) {
  if (!dtype_ok(dtype)) return fail(HYATTN_ERR_UNSUPPORTED, "dtype %d not supported", (int)dtype);
  if (!d_ok(D)) return fail(HYATTN_ERR_UNSUPPORTED, "head dim %d not supported (64 or 128)", D);
  if (B < 0) return fail(HYATTN_ERR_INVALID_ARG, "B = %d < 0", B);
  if (H_kv < 1 || H_q < 1 || H_q % H_kv != 0)
    return fail(HYATTN_ERR_INVALID_ARG, "H_q = %d must be a positive multiple of H_kv = %d", H_q,
                H_kv);
  if (n_blocks < 1 || max_blocks < 1)
    return fail(HYATTN_ERR_INVALID_ARG, "n_blocks and max_blocks_per_seq must be positive");
  return ok();
}

hyattn_status hyattn_paged_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                  int64_t n_blocks, const int32_t* bt, int max_blocks,
                                  const int32_t* ctx, const int32_t* cu_q, int B, int max_q_len,
                                  int H_kv, int D, hyattn_dtype dtype, void* stream) {
  hyattn_status st = check_full_dims(B, H_kv, H_kv, D, dtype, n_blocks, max_blocks);
  if (st != HYATTN_OK) return st;
  if (max_q_len < 0) return fail(HYATTN_ERR_INVALID_ARG, "max_q_len < 0");
  if (B == 0 || max_q_len == 0) return ok();
  if (!k_new || !v_new || !k_pool || !v_pool || !bt || !ctx || !cu_q)
    return fail(HYATTN_ERR_INVALID_ARG, "a pointer is NULL");
  hipStream_t s = as_stream(stream);
  if (checked_mode()) {
    std::vector<int32_t> cu, c;
    if ((st = fetch(cu, cu_q, (size_t)B + 1, s)) != HYATTN_OK) return st;
    if ((st = check_cu(cu, max_q_len, "cu_q_lens")) != HYATTN_OK) return st;
    if ((st = check_tables(bt, B, max_blocks, ctx, max_blocks * 16, n_blocks, s, &c)) != HYATTN_OK)
      return st;
    for (int r = 0; r < B; ++r)
      if (cu[r + 1] - cu[r] > c[r])
        return fail(HYATTN_ERR_INVALID_ARG, "request %d: %d new tokens > context %d", r,
                    cu[r + 1] - cu[r], c[r]);
  }
  return hip_status(hy::launch_paged_append(k_new, v_new, k_pool, v_pool, n_blocks, bt, max_blocks,
                                            ctx, cu_q, B, max_q_len, H_kv, D,
                                            dtype == HYATTN_BF16, s),
                    "paged append launch");
}

size_t hyattn_paged_decode_workspace_bytes(int B, int H_q, int D, int max_context) {
  if (B < 0 || H_q < 0 || D < 0 || max_context < 0) return 0;
  return hy::decode_workspace_bytes(B, H_q, D, max_context);
}

// Arguments of a decode call other than its workspace (and, in checked mode,
// the tables and context lengths).
static hyattn_status paged_decode_args(const void* q, const void* o, const void* k_pool,
                                       const void* v_pool, int64_t n_blocks, const int32_t* bt,
                                       int max_blocks, const int32_t* ctx, int max_context, int B,
                                       int H_q, int H_kv, int D, hyattn_dtype dtype,
                                       hipStream_t s) {
  hyattn_status st = check_full_dims(B, H_q, H_kv, D, dtype, n_blocks, max_blocks);
  if (st != HYATTN_OK) return st;
  if (max_context < 0 || (int64_t)max_context > (int64_t)max_blocks * 16)
    return fail(HYATTN_ERR_INVALID_ARG, "max_context %d outside [0, 16 * max_blocks_per_seq]",
                max_context);
  if (dtype == HYATTN_BF16 && H_q / H_kv != 1 && H_q / H_kv != 2 && H_q / H_kv != 4 &&
      H_q / H_kv != 8)
    return fail(HYATTN_ERR_UNSUPPORTED, "query heads per KV head must be 1, 2, 4 or 8 (got %d)",
                H_q / H_kv);
  if (B == 0) return ok();
  if (!q || !o || !k_pool || !v_pool || !bt || !ctx)
    return fail(HYATTN_ERR_INVALID_ARG, "a pointer is NULL");
  if (checked_mode() &&
      (st = check_tables(bt, B, max_blocks, ctx, max_context, n_blocks, s)) != HYATTN_OK)
    return st;
  return ok();
}

hyattn_status hyattn_paged_decode(const void* q, void* o, const void* k_pool, const void* v_pool,
                                  int64_t n_blocks, const int32_t* bt, int max_blocks,
                                  const int32_t* ctx, int max_context, int B, int H_q, int H_kv,
                                  int D, float scale, void* workspace, size_t workspace_bytes,
                                  hyattn_dtype dtype, void* stream) {
  hipStream_t s = as_stream(stream);
  hyattn_status st = paged_decode_args(q, o, k_pool, v_pool, n_blocks, bt, max_blocks, ctx,
                                       max_context, B, H_q, H_kv, D, dtype, s);
  if (st != HYATTN_OK || B == 0) return st;
  const size_t need = hy::decode_workspace_bytes(B, H_q, D, max_context);
  if (dtype == HYATTN_BF16 && (!workspace || workspace_bytes < need))
    return fail(HYATTN_ERR_INVALID_ARG, "workspace needs %zu bytes (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  return hip_status(hy::launch_paged_decode(q, o, k_pool, v_pool, n_blocks, bt, max_blocks, ctx,
                                            max_context, B, H_q, H_kv, D, scale, workspace,
                                            dtype == HYATTN_BF16, s),
                    "paged decode launch");
}

hyattn_status hyattn_paged_decode_noalloc(const void* q, void* o, const void* k_pool,
                                          const void* v_pool, int64_t n_blocks, const int32_t* bt,
                                          int max_blocks, const int32_t* ctx, int max_context,
                                          int B, int H_q, int H_kv, int D, float scale,
                                          hyattn_dtype dtype, void* stream) {
  hipStream_t s = as_stream(stream);
  hyattn_status st = paged_decode_args(q, o, k_pool, v_pool, n_blocks, bt, max_blocks, ctx,
                                       max_context, B, H_q, H_kv, D, dtype, s);
  if (st != HYATTN_OK || B == 0) return st;
  void* ws = nullptr;
  if (dtype == HYATTN_BF16) {
    const size_t need = hy::decode_launch_bytes(B, H_q, H_kv, D, max_context);
    if (need > hy::kDecodeScratchBytes)
      return fail(HYATTN_ERR_INVALID_ARG,
                  "decode of B=%d, H_q=%d, D=%d, max_context=%d needs %zu bytes of scratch; the "
                  "allocation-free entry point holds %zu (use hyattn_paged_decode with a workspace)",
                  B, H_q, D, max_context, need, hy::kDecodeScratchBytes);
    hipError_t e = hy::decode_scratch(&ws);
    if (e != hipSuccess) return hip_status(e, "looking up the decode scratch array");
  }
  return hip_status(hy::launch_paged_decode(q, o, k_pool, v_pool, n_blocks, bt, max_blocks, ctx,
                                            max_context, B, H_q, H_kv, D, scale, ws,
                                            dtype == HYATTN_BF16, s),
                    "paged decode launch");
}

hyattn_status hyattn_paged_prefill(const void* q, void* o, const void* k_pool, const void* v_pool,
                                   int64_t n_blocks, const int32_t* bt, int max_blocks,
                                   const int32_t* ctx, const int32_t* cu_q, int max_q_len, int B,
                                   int H_q, int H_kv, int D, float scale, hyattn_dtype dtype,
                                   void* stream) {
  hyattn_status st = check_full_dims(B, H_q, H_kv, D, dtype, n_blocks, max_blocks);
  if (st != HYATTN_OK) return st;
  if (max_q_len < 0) return fail(HYATTN_ERR_INVALID_ARG, "max_q_len < 0");
  if (B == 0 || max_q_len == 0) return ok();
  if (!q || !o || !k_pool || !v_pool || !bt || !ctx || !cu_q)
    return fail(HYATTN_ERR_INVALID_ARG, "a pointer is NULL");
  hipStream_t s = as_stream(stream);
  if (checked_mode()) {
    std::vector<int32_t> cu, c;
    if ((st = fetch(cu, cu_q, (size_t)B + 1, s)) != HYATTN_OK) return st;
    if ((st = check_cu(cu, max_q_len, "cu_q_lens")) != HYATTN_OK) return st;
    if ((st = check_tables(bt, B, max_blocks, ctx, max_blocks * 16, n_blocks, s, &c)) != HYATTN_OK)
      return st;
    for (int r = 0; r < B; ++r)
      if (cu[r + 1] - cu[r] > c[r])
        return fail(HYATTN_ERR_INVALID_ARG, "request %d: %d queries > context %d", r,
                    cu[r + 1] - cu[r], c[r]);
  }
  return hip_status(hy::launch_paged_prefill(q, o, k_pool, v_pool, n_blocks, bt, max_blocks, ctx, cu_q,
                                             max_q_len, B, H_q, H_kv, D, scale,
                                             dtype == HYATTN_BF16, s),
                    "paged prefill launch");
}

// ---------------------------------------------------------------- hybrid step --
hyattn_status hyattn_estimate_memory(const int32_t* layer_types, int n_layers, int H, int H_kv,
                                     int D, const int32_t* context_lens, int n_requests,
                                     int kv_elem_bytes, int state_elem_bytes,
                                     hyattn_memory_estimate* out) {
  if (!out) return fail(HYATTN_ERR_INVALID_ARG, "out is NULL");
  if (n_layers < 0 || n_requests < 0 || H < 0 || H_kv < 0 || D < 0 || kv_elem_bytes < 0 ||
      state_elem_bytes < 0)
    return fail(HYATTN_ERR_INVALID_ARG, "negative size");
  if ((n_layers > 0 && !layer_types) || (n_requests > 0 && !context_lens))
    return fail(HYATTN_ERR_INVALID_ARG, "layer_types or context_lens is NULL");
  int n_full = 0, n_lin = 0;
  for (int i = 0; i < n_layers; ++i) {
    if (layer_types[i] == HYATTN_LAYER_FULL)
      ++n_full;
    else if (layer_types[i] == HYATTN_LAYER_LINEAR)
      ++n_lin;
    else
      return fail(HYATTN_ERR_UNSUPPORTED_LAYER, "layer %d: attention type %d is not supported", i,
                  layer_types[i]);
  }
  typedef unsigned __int128 u128;
  u128 tokens = 0, blocks = 0;
  for (int r = 0; r < n_requests; ++r) {
    if (context_lens[r] < 0) return fail(HYATTN_ERR_INVALID_ARG, "context_lens[%d] < 0", r);
    tokens += (u128)context_lens[r];
    blocks += ((u128)context_lens[r] + HYATTN_BLOCK_TOKENS - 1) / HYATTN_BLOCK_TOKENS;
  }
  const u128 per_token = (u128)2 * (unsigned)n_full * (unsigned)H_kv * (unsigned)D * (unsigned)kv_elem_bytes;
  const u128 kv = per_token * tokens;
  const u128 kv_paged = per_token * blocks * HYATTN_BLOCK_TOKENS;
  const u128 state = (u128)(unsigned)n_lin * (unsigned)H * (unsigned)D * (unsigned)D *
                     (unsigned)n_requests * (unsigned)state_elem_bytes;
  const u128 lim = (u128)UINT64_MAX;
  if (kv > lim || kv_paged > lim || state > lim || blocks > lim)
    return fail(HYATTN_ERR_INVALID_ARG, "estimate exceeds 2^64 - 1 bytes");
  out->kv_bytes = (uint64_t)kv;
  out->kv_paged_bytes = (uint64_t)kv_paged;
  out->kv_blocks = (uint64_t)blocks;
  out->state_bytes = (uint64_t)state;
  out->n_full_layers = n_full;
  out->n_linear_layers = n_lin;
  return ok();
}

hyattn_status hyattn_bucket_by_length(const int32_t* lengths, int n, int64_t max_padded_tokens,
                                      int max_requests, int32_t* order, int32_t* batch_offsets,
                                      int* n_batches) {
  if (n < 0) return fail(HYATTN_ERR_INVALID_ARG, "n < 0");
  if (!n_batches || !batch_offsets || (n > 0 && (!lengths || !order)))
    return fail(HYATTN_ERR_INVALID_ARG, "NULL argument");
  if (max_padded_tokens < 1 || max_requests < 1)
    return fail(HYATTN_ERR_INVALID_ARG, "max_padded_tokens and max_requests must be >= 1");
  for (int r = 0; r < n; ++r) {
    if (lengths[r] < 0) return fail(HYATTN_ERR_INVALID_ARG, "lengths[%d] < 0", r);
    if (lengths[r] > max_padded_tokens)
      return fail(HYATTN_ERR_INVALID_ARG, "request %d: %d tokens exceed max_padded_tokens %lld", r,
                  lengths[r], (long long)max_padded_tokens);
  }
  std::vector<int32_t> idx(n);
  for (int r = 0; r < n; ++r) idx[r] = r;
  std::stable_sort(idx.begin(), idx.end(),
                   [&](int32_t a, int32_t b) { return lengths[a] < lengths[b]; });
  // Sorted ascending, the request being added is always the batch's longest.
  std::vector<int32_t> offs{0};
  int64_t count = 0;
  for (int i = 0; i < n; ++i) {
    const int64_t len = lengths[idx[i]];
    if (count > 0 && (count + 1 > max_requests || (count + 1) * len > max_padded_tokens)) {
      offs.push_back(i);
      count = 0;
    }
    ++count;
  }
  if (n > 0) offs.push_back(n);
  for (int i = 0; i < n; ++i) order[i] = idx[i];
  for (size_t b = 0; b < offs.size(); ++b) batch_offsets[b] = offs[b];
  *n_batches = (int)offs.size() - 1;
  return ok();
}

size_t hyattn_hybrid_workspace_bytes(const hyattn_batch* b) {
  if (!b || b->n_decode < 0) return 0;
  return hy::decode_workspace_bytes(b->n_decode, b->H, b->D, b->max_context);
}

// Checked mode for the hybrid step: every index array of the batch is read once
// and validated before the step launches anything.
static hyattn_status check_step_contents(const hyattn_batch* b, hyattn_state_pool* p, int n_lin,
                                         int n_full, const int32_t* layer_types, int n_layers,
                                         const hyattn_layer_io* layers, hipStream_t s) {
  const int B = b->n_prefill + b->n_decode;
  hyattn_status st;
  std::vector<int32_t> cu_p;
  if (b->n_prefill > 0) {
    if ((st = fetch(cu_p, b->cu_seqlens, (size_t)b->n_prefill + 1, s)) != HYATTN_OK) return st;
    if ((st = check_cu(cu_p, b->max_prefill_len, "cu_seqlens")) != HYATTN_OK) return st;
    if (cu_p[b->n_prefill] != b->n_prefill_tokens)
      return fail(HYATTN_ERR_INVALID_ARG, "cu_seqlens[%d] = %d but n_prefill_tokens = %d",
                  b->n_prefill, cu_p[b->n_prefill], b->n_prefill_tokens);
  }
  if (n_lin > 0) {
    // prefill and decode slots together: allocated, zeroed since allocation, no repeats
    std::vector<int32_t> sp, sd;
    if (b->n_prefill > 0 && (st = fetch(sp, b->prefill_slots, (size_t)b->n_prefill, s)) != HYATTN_OK)
      return st;
    if (b->n_decode > 0 && (st = fetch(sd, b->decode_slots, (size_t)b->n_decode, s)) != HYATTN_OK)
      return st;
    sp.insert(sp.end(), sd.begin(), sd.end());
    std::lock_guard<std::mutex> lk(p->mu);
    std::vector<unsigned char> seen(p->n_slots, 0);
    for (size_t i = 0; i < sp.size(); ++i) {
      const int id = sp[i];
      if (id < 0 || id >= p->n_slots)
        return fail(HYATTN_ERR_BAD_SLOT, "slot %d (request %zu) outside [0, %d)", id, i, p->n_slots);
      if (!p->used[id]) return fail(HYATTN_ERR_BAD_SLOT, "slot %d (request %zu) is not allocated", id, i);
      if (!p->zeroed[id])
        return fail(HYATTN_ERR_BAD_SLOT, "slot %d (request %zu) was never zeroed since allocation", id, i);
      if (seen[id]) return fail(HYATTN_ERR_INVALID_ARG, "slot %d serves two requests of the step", id);
      seen[id] = 1;
    }
  }
  for (int i = 0; i < n_layers; ++i)
    if (layer_types[i] == HYATTN_LAYER_LINEAR && layers[i].log_gamma &&
        (st = check_log_gamma(layers[i].log_gamma,
                              ((size_t)(b->n_prefill > 0 ? b->n_prefill_tokens : 0) + b->n_decode) * b->H,
                              s)) != HYATTN_OK)
      return st;
  if (n_full > 0) {
    std::vector<int32_t> cu_q, c;
    if ((st = fetch(cu_q, b->cu_q_lens, (size_t)B + 1, s)) != HYATTN_OK) return st;
    for (int r = 0; r <= B; ++r) {  // cu_seqlens, then one row per decode request
      const int want = r <= b->n_prefill ? (b->n_prefill > 0 ? cu_p[r] : 0)
                                         : (b->n_prefill > 0 ? cu_p[b->n_prefill] : 0) + r - b->n_prefill;
      if (cu_q[r] != want)
        return fail(HYATTN_ERR_INVALID_ARG, "cu_q_lens[%d] = %d, expected %d", r, cu_q[r], want);
    }
    if ((st = check_tables(b->block_tables, B, b->max_blocks_per_seq, b->context_lens,
                           b->max_context, b->n_blocks, s, &c)) != HYATTN_OK)
      return st;
    for (int r = 0; r < B; ++r)
      if (cu_q[r + 1] - cu_q[r] > c[r])
        return fail(HYATTN_ERR_INVALID_ARG, "request %d: %d new tokens > context %d", r,
                    cu_q[r + 1] - cu_q[r], c[r]);
  }
  return ok();
}

hyattn_status hyattn_hybrid_step(const int32_t* layer_types, int n_layers,
                                 const hyattn_layer_io* layers, const hyattn_batch* b,
                                 hyattn_state_pool* p, void* stream) {
  if (n_layers < 0) return fail(HYATTN_ERR_INVALID_ARG, "n_layers < 0");
  if (n_layers > 0 && (!layer_types || !layers))
    return fail(HYATTN_ERR_INVALID_ARG, "layer_types or layers is NULL");
  if (!b) return fail(HYATTN_ERR_INVALID_ARG, "batch is NULL");
  // 1. every layer type is known (P1 §4.3: unknown attention types are rejected)
  int n_lin = 0, n_full = 0;
  for (int i = 0; i < n_layers; ++i) {
    if (layer_types[i] == HYATTN_LAYER_LINEAR)
      ++n_lin;
    else if (layer_types[i] == HYATTN_LAYER_FULL)
      ++n_full;
    else
      return fail(HYATTN_ERR_UNSUPPORTED_LAYER, "layer %d: attention type %d is not supported", i,
                  layer_types[i]);
  }
  // 2. every argument of every layer, before any launch: a step that fails has
  //    no side effects (no linear state advanced, no token appended)
  if (b->n_prefill < 0 || b->n_decode < 0)
    return fail(HYATTN_ERR_INVALID_ARG, "negative request counts");
  const int B = b->n_prefill + b->n_decode;
  if (!dtype_ok(b->dtype)) return fail(HYATTN_ERR_UNSUPPORTED, "dtype %d not supported", b->dtype);
  if (b->n_prefill > 0) {
    if (!b->cu_seqlens) return fail(HYATTN_ERR_INVALID_ARG, "prefill requests need cu_seqlens");
    if (b->n_prefill_tokens < 0 || b->max_prefill_len < 0)
      return fail(HYATTN_ERR_INVALID_ARG, "n_prefill_tokens and max_prefill_len must be >= 0");
  }
  const bool bf16 = b->dtype == HYATTN_BF16;
  if (n_lin > 0) {
    if (!p) return fail(HYATTN_ERR_INVALID_ARG, "linear layers need a state pool");
    if (n_lin > p->n_layers)
      return fail(HYATTN_ERR_INVALID_ARG, "%d linear layers but the pool holds %d", n_lin,
                  p->n_layers);
    if (p->H != b->H || p->D != b->D)
      return fail(HYATTN_ERR_INVALID_ARG, "pool (H=%d, D=%d) does not match batch (H=%d, D=%d)",
                  p->H, p->D, b->H, b->D);
    if (b->n_prefill > 0 && !b->prefill_slots)
      return fail(HYATTN_ERR_INVALID_ARG, "prefill requests need slots");
    if (b->n_decode > 0 && !b->decode_slots)
      return fail(HYATTN_ERR_INVALID_ARG, "decode requests need slots");
    bool any_gated = false;
    for (int i = 0; i < n_layers; ++i)
      any_gated |= layer_types[i] == HYATTN_LAYER_LINEAR && layers[i].log_gamma != nullptr;
    if (b->n_prefill > 0 && !prefill_chunk_ok(b->D, b->chunk_size, b->dtype, any_gated))
      return fail(HYATTN_ERR_UNSUPPORTED, "chunk_size %d not supported", b->chunk_size);
  }
  if (n_full > 0) {
    hyattn_status st = check_full_dims(B, b->H, b->H_kv, b->D, b->dtype, b->n_blocks,
                                       b->max_blocks_per_seq);
    if (st != HYATTN_OK) return st;
    if (!b->block_tables || !b->context_lens || !b->cu_q_lens)
      return fail(HYATTN_ERR_INVALID_ARG, "full layers need block tables, context and q lengths");
    if (b->max_context < 0 || (int64_t)b->max_context > (int64_t)b->max_blocks_per_seq * 16)
      return fail(HYATTN_ERR_INVALID_ARG, "max_context %d outside [0, 16 * max_blocks_per_seq]",
                  b->max_context);
    const int G = b->H / b->H_kv;
    if (bf16 && G != 1 && G != 2 && G != 4 && G != 8)
      return fail(HYATTN_ERR_UNSUPPORTED, "query heads per KV head must be 1, 2, 4 or 8 (got %d)", G);
    if (b->n_decode > 0) {
      const size_t need = hy::decode_workspace_bytes(b->n_decode, b->H, b->D, b->max_context);
      if (bf16 && (!b->workspace || b->workspace_bytes < need))
        return fail(HYATTN_ERR_INVALID_ARG, "workspace needs %zu bytes", need);
    }
  }
  for (int i = 0; i < n_layers; ++i) {
    const hyattn_layer_io& L = layers[i];
    if (B > 0 && (!L.q || !L.k || !L.v || !L.o))
      return fail(HYATTN_ERR_INVALID_ARG, "layer %d: q/k/v/o pointer is NULL", i);
    if (layer_types[i] == HYATTN_LAYER_FULL && (!L.k_pool || !L.v_pool))
      return fail(HYATTN_ERR_INVALID_ARG, "layer %d: full layer without KV pools", i);
    if (layer_types[i] == HYATTN_LAYER_FULL && L.log_gamma)
      return fail(HYATTN_ERR_INVALID_ARG, "layer %d: log_gamma is for linear layers only", i);
  }
  if (B == 0) return ok();
  hipStream_t s = as_stream(stream);
  if (checked_mode()) {
    hyattn_status st = check_step_contents(b, p, n_lin, n_full, layer_types, n_layers, layers, s);
    if (st != HYATTN_OK) return st;
  }
  if (getenv("HYATTN_LOG")) {
    std::string plan;
    for (int i = 0; i < n_layers; ++i) plan += layer_types[i] == HYATTN_LAYER_LINEAR ? 'L' : 'F';
    fprintf(stderr, "[hyattn] step: %d layers (%d linear, %d full) plan %s; %d prefill + %d decode\n",
            n_layers, n_lin, n_full, plan.c_str(), b->n_prefill, b->n_decode);
  }
  // 3. launches in layer order (arguments validated above). A full layer with
  //    both prefill and decode requests forks its decode attention onto the
  //    side stream after the append and joins it back before the next layer.
  const bool fork_full = n_full > 0 && b->n_prefill > 0 && b->max_prefill_len > 0 && b->n_decode > 0;
  SideStream* side = nullptr;
  int n_cus = 0;
  if (fork_full) {
    hipError_t e = side_stream(&side);
    if (e == hipSuccess) e = hy::device_cus(&n_cus);
    if (e != hipSuccess) return hip_status(e, "hybrid step side stream");
  }
  const size_t esz = bf16 ? 2 : 4;
  // every full layer's decode serves the same requests: their work-item layout
  // is computed once, here, and each decode launch reuses it from the workspace
  const bool plan_once = n_full > 0 && b->n_decode > 0 && bf16;
  if (plan_once) {
    hipError_t e = hy::launch_decode_plan(b->context_lens + b->n_prefill, b->max_context,
                                          b->n_decode, b->H, b->H_kv, b->D,
                                          b->max_blocks_per_seq, b->workspace, s);
    if (e != hipSuccess) return hip_status(e, "hybrid step decode plan");
  }
  const int n_prefill_tok = b->n_prefill > 0 ? b->n_prefill_tokens : 0;
  const size_t off = (size_t)n_prefill_tok * b->H * b->D * esz;  // first decode row
  const int max_q_len = b->n_prefill > 0 ? std::max(b->max_prefill_len, 1) : 1;
  int li = 0;
  for (int i = 0; i < n_layers; ++i) {
    const hyattn_layer_io& L = layers[i];
    hipError_t e = hipSuccess;
    if (layer_types[i] == HYATTN_LAYER_LINEAR) {
      float* base = layer_base(p, li++);
      if (b->n_prefill > 0)
        e = hy::launch_linear_prefill(base, p->n_slots, L.q, L.k, L.v, L.o, L.log_gamma,
                                      b->cu_seqlens, b->prefill_slots, b->n_prefill, b->H, b->D,
                                      b->chunk_size, bf16, s);
      if (e == hipSuccess && b->n_decode > 0)
        e = hy::launch_linear_decode(base, p->n_slots, (const char*)L.q + off,
                                     (const char*)L.k + off, (const char*)L.v + off,
                                     (char*)L.o + off,
                                     L.log_gamma ? L.log_gamma + (size_t)n_prefill_tok * b->H : nullptr,
                                     b->decode_slots, b->n_decode, b->H, b->D, bf16, s);
    } else {
      e = hy::launch_paged_append(L.k, L.v, L.k_pool, L.v_pool, b->n_blocks, b->block_tables,
                                  b->max_blocks_per_seq, b->context_lens, b->cu_q_lens, B,
                                  max_q_len, b->H_kv, b->D, bf16, s);
      auto decode = [&](hipStream_t ds) {
        return hy::launch_paged_decode((const char*)L.q + off, (char*)L.o + off, L.k_pool,
                                       L.v_pool, b->n_blocks,
                                       b->block_tables + (size_t)b->n_prefill * b->max_blocks_per_seq,
                                       b->max_blocks_per_seq, b->context_lens + b->n_prefill,
                                       b->max_context, b->n_decode, b->H, b->H_kv, b->D, b->scale,
                                       b->workspace, bf16, ds, plan_once);
      };
      auto prefill = [&](int grid_cap) {
        return hy::launch_paged_prefill(L.q, L.o, L.k_pool, L.v_pool, b->n_blocks, b->block_tables,
                                        b->max_blocks_per_seq, b->context_lens, b->cu_seqlens,
                                        b->max_prefill_len, b->n_prefill, b->H, b->H_kv, b->D,
                                        b->scale, bf16, s, grid_cap);
      };
      if (e == hipSuccess && fork_full) {
        // decode on the side stream (after the append), prefill here, then join
        std::lock_guard<std::mutex> lk(side->mu);
        if ((e = hipEventRecord(side->fork, s)) == hipSuccess &&
            (e = hipStreamWaitEvent(side->s, side->fork, 0)) == hipSuccess) {
          // beside the decode the prefill runs one persistent workgroup per CU,
          // so that every CU keeps room for decode workgroups
          const hipError_t ed = decode(side->s);
          const hipError_t ep = ed == hipSuccess ? prefill(n_cus) : hipSuccess;
          // joined whatever the launches returned, so that all side-stream
          // work is ordered before anything the caller queues next
          e = hipEventRecord(side->join, side->s);
          if (e == hipSuccess) e = hipStreamWaitEvent(s, side->join, 0);
          if (e == hipSuccess) e = ed != hipSuccess ? ed : ep;
        }
      } else {
        if (e == hipSuccess && b->n_prefill > 0 && b->max_prefill_len > 0) e = prefill(0);
        if (e == hipSuccess && b->n_decode > 0) e = decode(s);
      }
    }
    if (e != hipSuccess) return hip_status(e, "hybrid step launch");
  }
  return ok();
}

}  // extern "C"
