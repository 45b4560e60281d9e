// Host-side launchers of the hyattn gfx950 kernels (internal to the library).
// Each launcher assumes its arguments were validated by the C-ABI layer and
// returns the hipError_t of the launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hy {

// ---- linear layers ------------------------------------------------------------
hipError_t launch_state_zero(float* pool, int n_layers, int n_slots, int64_t slot_elems,
                             const int32_t* slots, int n, hipStream_t s);

// log_gamma: NULL for the plain layer, else the gated variant's per-token log
// forget factors, fp32 [N_tok][H] (decode: [B][H]).
hipError_t launch_linear_decode(float* layer_states, int n_slots, const void* q, const void* k,
                                const void* v, void* o, const float* log_gamma,
                                const int32_t* slots, int B, int H, int D, bool bf16,
                                hipStream_t s);

hipError_t launch_linear_prefill(float* layer_states, int n_slots, const void* q, const void* k,
                                 const void* v, void* o, const float* log_gamma,
                                 const int32_t* cu, const int32_t* slots, int n_req, int H, int D,
                                 int chunk, bool bf16, hipStream_t s);

// LDS bytes of the bf16 prefill kernel at chunk size C (plain or gated).
size_t linear_prefill_bf16_lds_bytes(int D, int C, bool gated);

// Largest chunk the fp32-I/O prefill kernel takes (its chunk scores live in LDS).
constexpr int kMaxChunkF32 = 128;

// Compute units of the current device (cached per device).
hipError_t device_cus(int* out);

// ---- full layers --------------------------------------------------------------
hipError_t launch_paged_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                               int64_t n_blocks, const int32_t* bt, int max_blocks,
                               const int32_t* ctx, const int32_t* cu_q, int B, int max_q_len,
                               int H_kv, int D, bool bf16, hipStream_t s);

struct DecodePlan {
  int part_blocks;  // 16-token blocks per context partition
  int max_parts;    // partitions of the longest context
};
// work_pairs = B x H_kv of the launch (0: no floor, the most partitions, which
// sizes the workspace)
DecodePlan decode_plan(int max_context, int64_t work_pairs);
size_t decode_workspace_bytes(int B, int H_q, int D, int max_context);
// bytes of workspace one launch_paged_decode call of these sizes uses
size_t decode_launch_bytes(int B, int H_q, int H_kv, int D, int max_context);
// Device address of this device's scratch array (kDecodeScratchBytes), looked
// up on the first call on each device; the allocation-free decode uses it as
// its workspace.
constexpr size_t kDecodeScratchBytes = (size_t)64 << 20;
hipError_t decode_scratch(void** out);

// plan_ready: the work-item layout of these (ctx, max_context, B, H_q, H_kv, D,
// max_blocks) already sits in `workspace` (launch_decode_plan, or an earlier
// decode of the same requests on the same stream order), so the call skips it.
hipError_t launch_paged_decode(const void* q, void* o, const void* k_pool, const void* v_pool,
                               int64_t n_blocks, const int32_t* bt, int max_blocks,
                               const int32_t* ctx, int max_context,
                               int B, int H_q, int H_kv, int D, float scale, void* workspace,
                               bool bf16, hipStream_t s, bool plan_ready = false);
// The work-item layout of a bf16 decode of these requests into `workspace`,
// as launch_paged_decode lays it out first.
hipError_t launch_decode_plan(const int32_t* ctx, int max_context, int B, int H_q, int H_kv, int D,
                              int max_blocks, void* workspace, hipStream_t s);

// VALU paged attention for fp32 I/O (decode with cu_q = NULL, or causal prefill).
hipError_t launch_paged_simple_f32(const void* q, void* o, const void* k_pool, const void* v_pool,
                                   int64_t n_blocks, const int32_t* bt, int max_blocks,
                                   const int32_t* ctx, const int32_t* cu_q, int max_q_len, int B,
                                   int H_q, int H_kv, int D, float scale, hipStream_t s);

// grid_cap > 0 (bf16): at most that many workgroups, each walking several
// query tiles (the hybrid step passes the CU count when the layer's decode runs
// beside the prefill, so that every CU keeps room for decode workgroups).
hipError_t launch_paged_prefill(const void* q, void* o, const void* k_pool, const void* v_pool,
                                int64_t n_blocks, const int32_t* bt, int max_blocks,
                                const int32_t* ctx,
                                const int32_t* cu_q, int max_q_len, int B, int H_q, int H_kv,
                                int D, float scale, bool bf16, hipStream_t s, int grid_cap = 0);

}  // namespace hy
