// Full-attention kernels over a paged KV cache of 16-token blocks for gfx950:
// KV append, split-context decode with a log-sum-exp merge, and the VALU path
// for fp32 I/O (decode and causal prefill). The bf16 causal prefill is in
// k_prefill.hip.
//
// Method (page "推理框架适配Hybrid Model：KV Cache管理与算子调度实战", "P2"):
//   §2.1  KV is cut into fixed 16-token blocks mapped through a per-request
//         page (block) table; full-attention decode costs O(S * D) per token.
//   §2.3  decode is PagedAttention over Q, K, V and the block table; prefill a
//         FlashAttention-class kernel.
// Layout: pool [n_blocks][H_kv][16][D]; logical token p of request r lives in
// block bt[r][p / 16] at offset p % 16; query head h reads KV head
// h / (H_q / H_kv). Softmax is evaluated in base 2 on scores pre-multiplied by
// scale * log2(e), with the running maximum subtracted (fp32 throughout).
#include <math.h>

#include <mutex>

#include "hy_common.hpp"
#include "hy_kernels.hpp"

namespace hy {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescale = 8.f;  // log2 headroom before the softmax reference moves
constexpr float kRescaleSum = 65536.f;     // bound on a lane's p-sum before the reference moves
constexpr float kMinusHuge = -0x1p100f;    // finite stand-in for -inf as a softmax reference
constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;  // bf16 pair (1, 1)

// ============================================================================
// Append: copy each new token's K and V rows into its slot. grid (token tiles
// of 16, B); 16-byte vector copies.
// ============================================================================
template <typename T>
__global__ __launch_bounds__(256) void k_paged_append(const T* __restrict__ k_new,
                                                      const T* __restrict__ v_new,
                                                      T* __restrict__ k_pool, T* __restrict__ v_pool,
                                                      int64_t n_blocks, const int32_t* __restrict__ bt,
                                                      int max_blocks, const int32_t* __restrict__ ctx,
                                                      const int32_t* __restrict__ cu, int H_kv, int D) {
  constexpr int VEC = 16 / sizeof(T);
  const int r = blockIdx.y;
  const int q0 = cu[r], ql = cu[r + 1] - q0;
  const int c = ctx[r];
  const int vec_per_tok = H_kv * D / VEC;
  const int tok_begin = blockIdx.x * 16;
  for (int idx = threadIdx.x; idx < 16 * vec_per_tok; idx += 256) {
    const int i = tok_begin + idx / vec_per_tok;
    if (i >= ql) break;
    const int e = (idx % vec_per_tok) * VEC;  // element within [H_kv][D]
    const int g = e / D, d = e - (e / D) * D;
    const int p = c - ql + i;
    if (p < 0 || (p >> 4) >= max_blocks) continue;
    const int32_t blk = bt[(int64_t)r * max_blocks + (p >> 4)];
    if (blk < 0 || blk >= n_blocks) continue;
    const int64_t dst = (((int64_t)blk * H_kv + g) * kBlock + (p & 15)) * D + d;
    const int64_t src = ((int64_t)(q0 + i) * H_kv + g) * D + d;
    *reinterpret_cast<u32x4*>(k_pool + dst) = *reinterpret_cast<const u32x4*>(k_new + src);
    *reinterpret_cast<u32x4*>(v_pool + dst) = *reinterpret_cast<const u32x4*>(v_new + src);
  }
}

hipError_t launch_paged_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                               int64_t n_blocks, const int32_t* bt, int max_blocks,
                               const int32_t* ctx, const int32_t* cu_q, int B, int max_q_len,
                               int H_kv, int D, bool bf16, hipStream_t s) {
  if (B <= 0 || max_q_len <= 0) return hipSuccess;
  dim3 grid((unsigned)((max_q_len + 15) / 16), (unsigned)B), block(256);
  if (bf16)
    hipLaunchKernelGGL(k_paged_append<uint16_t>, grid, block, 0, s, (const uint16_t*)k_new,
                       (const uint16_t*)v_new, (uint16_t*)k_pool, (uint16_t*)v_pool, n_blocks, bt,
                       max_blocks, ctx, cu_q, H_kv, D);
  else
    hipLaunchKernelGGL(k_paged_append<float>, grid, block, 0, s, (const float*)k_new,
                       (const float*)v_new, (float*)k_pool, (float*)v_pool, n_blocks, bt,
                       max_blocks, ctx, cu_q, H_kv, D);
  return hipGetLastError();
}

// ============================================================================
// Decode planning: a request's context is split into partitions of
// part_blocks blocks (a multiple of 4 blocks = one pass of a workgroup, at
// most kMaxParts partitions for the longest context). Work items are the
// (request, partition) pairs; k_decode_plan lays them out with an exclusive
// scan, so the attention grid never holds empty workgroups.
//
// Each item starts its waves' load rings from empty and ends with a merge, so
// long partitions stream better: with work to spare, partitions are at least
// kPartFloor blocks (4096 tokens). The floor comes down when the work bound
// (B x H_kv x the longest context's blocks) would leave fewer than about
// kTargetItems items, so that a small batch still spreads over the chip.
// ============================================================================
constexpr int kPassBlocks = 4;  // blocks per workgroup step (4 waves x 1 block)
constexpr int kMaxParts = 64;
constexpr int kPartFloor = 256;
constexpr int64_t kTargetItems = 8192;

DecodePlan decode_plan(int max_context, int64_t work_pairs) {
  const int nblk = (max_context + kBlock - 1) / kBlock;
  int pb = (nblk + kMaxParts - 1) / kMaxParts;
  if (work_pairs > 0) {
    const int64_t fit = (work_pairs * nblk) / kTargetItems;
    const int floor_pb = (int)(fit < kPartFloor ? fit : kPartFloor);
    if (floor_pb > pb) pb = floor_pb;
  }
  pb = ((pb + kPassBlocks - 1) / kPassBlocks) * kPassBlocks;
  if (pb < kPassBlocks) pb = kPassBlocks;
  int parts = (nblk + pb - 1) / pb;
  if (parts < 1) parts = 1;
  return DecodePlan{pb, parts};
}

static size_t decode_partials_bytes(int B, int H_q, int D, int max_parts) {
  const size_t b = (size_t)B * H_q * max_parts * (size_t)(D + 2) * sizeof(float);
  return (b + 255) & ~(size_t)255;
}

size_t decode_workspace_bytes(int B, int H_q, int D, int max_context) {
  const DecodePlan p = decode_plan(max_context, 0);  // the most partitions any launch uses
  return decode_partials_bytes(B, H_q, D, p.max_parts) + ((size_t)(B + 1) * sizeof(int32_t) + 255) / 256 * 256;
}

size_t decode_launch_bytes(int B, int H_q, int H_kv, int D, int max_context) {
  const DecodePlan p = decode_plan(max_context, (int64_t)B * H_kv);  // as launch_paged_decode
  return decode_partials_bytes(B, H_q, D, p.max_parts) + ((size_t)(B + 1) * sizeof(int32_t) + 255) / 256 * 256;
}

// ============================================================================
// Scratch of the allocation-free decode entry point: the partition partials
// and the partition scan live in this file-scope device array instead of a
// caller's workspace. Each GPU the library runs on holds its own copy until
// the process ends. In host code the array's name is only a stand-in, so its
// device address is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that address is ever handed to kernels.
// ============================================================================
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

__device__ __forceinline__ int n_parts_of(int c, int max_blocks, int part_blocks, int max_parts) {
  c = min(c, max_blocks * kBlock);  // defensive: never read past the table
  const int nblk = (max(c, 0) + kBlock - 1) / kBlock;
  return min((nblk + part_blocks - 1) / part_blocks, max_parts);
}

// One workgroup of 1024 threads: cu_parts[r] = sum of partitions of requests < r.
__global__ __launch_bounds__(1024) void k_decode_plan(const int32_t* __restrict__ ctx, int B,
                                                      int max_blocks, int part_blocks,
                                                      int max_parts, int32_t* __restrict__ cu_parts) {
  __shared__ int32_t sums[1024];
  const int t = threadIdx.x;
  const int per = (B + 1023) / 1024;
  const int r0 = min(B, t * per), r1 = min(B, r0 + per);
  int acc = 0;
  for (int r = r0; r < r1; ++r) acc += n_parts_of(ctx[r], max_blocks, part_blocks, max_parts);
  sums[t] = acc;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = t >= off ? sums[t - off] : 0;
    __syncthreads();
    sums[t] += v;
    __syncthreads();
  }
  int base = t ? sums[t - 1] : 0;
  for (int r = r0; r < r1; ++r) {
    cu_parts[r] = base;
    base += n_parts_of(ctx[r], max_blocks, part_blocks, max_parts);
  }
  if (t == 1023) cu_parts[B] = sums[1023];
}

// ============================================================================
// Decode, bf16. 1-D grid over (KV head g, worker), worker fastest, 4 waves;
// each workgroup walks the (request, partition) items worker, worker +
// n_workers, ... for its KV head.
// Wave w of a workgroup takes blocks w, w + 4, ... of the partition.
//
// K and V blocks reach LDS through direct global-to-LDS loads (no registers
// hold data in flight), each wave keeping its own ring of 2 block slots:
// block j + 1 is requested once block j has landed and is used while block j
// is, and the waves never synchronise inside an item. A workgroup takes
// 72 KiB of LDS at D = 128 (64 KiB of rings), so two fit a CU (as many bytes
// in flight per CU as one workgroup with 4-slot rings, and as fast alone),
// and one fits beside a causal-prefill workgroup (64 KiB): the hybrid step
// runs a full layer's decode beside its prefill on a second stream.
//   scores: v_mfma_f32_16x16x32_bf16 with A = the 16 K rows of the block
//           (each lane's K fragment lands at its own LDS offset), B = the G
//           query heads padded to 16 columns; lane l holds keys 4*(l/16)+i
//           of head l%16, which is directly the B operand of P V below;
//   softmax: a lazy reference per head, as in causal prefill (the common
//           case needs no cross-lane work);
//   P V:    O^T += V^T P^T with v_mfma_f32_16x16x16_bf16, the V^T operand by
//           transposing reads of the row-major, chunk-swizzled V tile.
// The waves are merged by log-sum-exp at the end of the item.
// ============================================================================
constexpr int kDecodeRing = 2;  // block slots per wave
// Cache policy of the K/V block loads (sc0 | nt): every byte is read once per
// call, so the loads stream past the caches (measured 3-8 % faster than the
// default policy on the random block tables of the decode workload).
constexpr int kStreamLoad = 3;

template <int D>
constexpr size_t decode_lds_bytes() {
  return (size_t)4 * kDecodeRing * 2 * kBlock * D * sizeof(uint16_t);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int D, int G>
__global__ __launch_bounds__(256) void k_paged_decode_bf16(
    const uint16_t* __restrict__ q, uint16_t* __restrict__ o, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, int64_t n_blocks, const int32_t* __restrict__ bt,
    int max_blocks, const int32_t* __restrict__ ctx, int B, int H_q, int H_kv, float scale_log2,
    int part_blocks, int max_parts, float* __restrict__ ws, const int32_t* __restrict__ cu_parts) {
  constexpr int KS = D / 32;     // k steps of the scores
  constexpr int NDT = D / 16;    // 16-dim tiles of O^T
  constexpr int NW = 4;
  constexpr int NB = kDecodeRing;
  constexpr int CPT = D / 8;     // 16-byte chunks per token row
  constexpr int RPI = 64 / CPT;  // V rows per wave-wide 16-byte load
  constexpr int NVI = kBlock / RPI;
  constexpr int IPB = KS + NVI;  // loads per block
  constexpr int SLOT = 2 * kBlock * D;  // elements per slot: K then V
  extern __shared__ __align__(16) uint16_t dec_lds[];
  __shared__ float s_m[NW][G], s_l[NW][G];
  __shared__ __align__(16) float s_acc[NW][G][D];

  // 1-D grid, worker fastest: consecutive workgroups go to consecutive XCDs,
  // so with a worker count that is a multiple of 8 every head of an item
  // runs on the same XCD, whose address translations then cover only the
  // pool pages of its own items
  const int n_workers = (int)gridDim.x / H_kv;
  const int g = (int)blockIdx.x / n_workers;
  const int worker = (int)blockIdx.x - g * n_workers;
  const int total = cu_parts[B];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
  const int w_s = __builtin_amdgcn_readfirstlane(w);  // wave index, as a scalar
  uint16_t* ring = dec_lds + w_s * NB * SLOT;
  // even chunk XOR of V row t of a block (transposing reads of 8 rows x 2
  // chunks per 32 lanes hit distinct banks)
  auto vswz = [](int t) -> int { return D == 128 ? 2 * (t & 7) : 2 * ((t >> 1) & 3); };

  for (int item = worker; item < total; item += n_workers) {
    int lo = 0, hi = B;  // cu_parts[lo] <= item < cu_parts[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cu_parts[mid] <= item) lo = mid; else hi = mid;
    }
    const int r = lo;
    const int part = item - cu_parts[r];
    const int c = min(ctx[r], max_blocks * kBlock);
    const int nblk = (c + kBlock - 1) / kBlock;
    const int n_parts = n_parts_of(c, max_blocks, part_blocks, max_parts);
    const int b_begin = part * part_blocks;
    const int b_end = min(nblk, b_begin + part_blocks);
    const int nbw = max(0, (b_end - b_begin - w_s + NW - 1) / NW);  // this wave's blocks
    const int h0 = g * G;
    const int32_t* btr = bt + (int64_t)r * max_blocks;

    u32x4 qf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[s] = lr < G ? *reinterpret_cast<const u32x4*>(q + ((int64_t)r * H_q + h0 + lr) * D + 32 * s + 8 * lg)
                     : u32x4{0u, 0u, 0u, 0u};
    // the Q fragments land first, so no later wait for them drains the ring
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    f32x4 ot[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) ot[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = kMinusHuge, l_run = 0.f;  // head lr's reference and this lane's share of its sum

    // ---- block j of this wave: global block b = b_begin + w + 4 j ----
    auto table = [&](int j) -> int32_t {  // raw table entry, validated at use
      return j < nbw ? btr[b_begin + w_s + NW * j] : -1;
    };
    auto issue = [&](int j, int32_t blk) {
      if (blk < 0 || blk >= n_blocks) blk = 0;  // absent: any valid block, masked and cleared
      const uint16_t* kb = k_pool + ((int64_t)blk * H_kv + g) * kBlock * D;
      const uint16_t* vb = v_pool + ((int64_t)blk * H_kv + g) * kBlock * D;
      uint16_t* slot = ring + (j % NB) * SLOT;
      // K: load s puts lane l's score operand (key l % 16, dims 32 s + 8 (l / 16) + 0..7)
      // at its own 16 bytes of a 1 KiB piece
#pragma unroll
      for (int s = 0; s < KS; ++s)
        __builtin_amdgcn_global_load_lds(kb + lr * D + 32 * s + 8 * lg,
                                         (__attribute__((address_space(3))) void*)(slot + s * 512),
                                         16, 0, kStreamLoad);
      // V: row-major, chunk c of row t at position c ^ vswz(t)
#pragma unroll
      for (int i = 0; i < NVI; ++i) {
        const int t = RPI * i + l / CPT;
        const int x = vswz(t);  // (a call inside the builtin's arguments would break the host stub)
        __builtin_amdgcn_global_load_lds(vb + t * D + 8 * ((l % CPT) ^ x),
                                         (__attribute__((address_space(3))) void*)(slot + kBlock * D + i * 512),
                                         16, 0, kStreamLoad);
      }
    };
    auto ntok_of = [&](int j, int32_t blk) -> int {  // valid keys of block j
      if (blk < 0 || blk >= n_blocks) return 0;
      return min(kBlock, c - kBlock * (b_begin + w_s + NW * j));
    };

    int32_t blk_ring[NB];
#pragma unroll
    for (int i = 0; i < NB - 1; ++i) {
      blk_ring[i] = table(i);
      if (i < nbw) issue(i, blk_ring[i]);
    }
    blk_ring[NB - 1] = table(NB - 1);

    for (int j = 0; j < nbw; ++j) {
      // block j landed: with two slots no later block has been requested yet
      static_assert(NB == 2, "the wait below assumes a 2-slot ring");
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      const int32_t blk = blk_ring[0];
      const int ntok = ntok_of(j, blk);
      const uint16_t* kslot = ring + (j % NB) * SLOT;
      uint16_t* vslot = ring + (j % NB) * SLOT + kBlock * D;
      if (ntok < kBlock) {  // rows without a key meet P V with weight 0: make them finite
        for (int e = l; e < kBlock * CPT; e += 64)
          if (e / CPT >= ntok) *reinterpret_cast<u32x4*>(vslot + 8 * e) = u32x4{0u, 0u, 0u, 0u};
      }
      if (j + NB - 1 < nbw) issue(j + NB - 1, blk_ring[NB - 1]);
#pragma unroll
      for (int i = 0; i < NB - 1; ++i) blk_ring[i] = blk_ring[i + 1];
      blk_ring[NB - 1] = table(j + NB);

      // ---- scores ----
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(kslot + s * 512 + 8 * l);
        sc = mfma16x16x32(kf, qf[s], sc);
      }
      // ---- softmax over head lr's 4 keys in this lane ----
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = (lr < G && 4 * lg + i < ntok) ? sc[i] : -INFINITY;
      auto probs = [&](uint32_t& p01, uint32_t& p23) -> float {
        const float e0 = fast_exp2(__builtin_fmaf(x[0], scale_log2, -m_run));
        const float e1 = fast_exp2(__builtin_fmaf(x[1], scale_log2, -m_run));
        const float e2 = fast_exp2(__builtin_fmaf(x[2], scale_log2, -m_run));
        const float e3 = fast_exp2(__builtin_fmaf(x[3], scale_log2, -m_run));
        p01 = pack_bf16x2(e0, e1);
        p23 = pack_bf16x2(e2, e3);
        return dot2_bf16(p23, kOnesBf16x2, dot2_bf16(p01, kOnesBf16x2, 0.f));
      };
      uint32_t p01, p23;
      float ps = probs(p01, p23);
      if (__builtin_amdgcn_ballot_w64(!(ps <= kRescaleSum))) {
        float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float ms = mx * scale_log2;  // -inf when the head has no key in the block
        float corr = 1.f;
        if (ms > m_run) {
          corr = fast_exp2(m_run - ms);  // 0 on the head's first key
          l_run *= corr;
          m_run = ms;
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          ot[dt][0] *= corr;
          ot[dt][1] *= corr;
          ot[dt][2] *= corr;
          ot[dt][3] *= corr;
        }
        ps = probs(p01, p23);
      }
      l_run += ps;
      // ---- O^T += V^T P^T ----
      const u32x2 pb = {p01, p23};
      u32x4 vv[NDT / 2];
      {
        // source lane (lg, lr) addresses key row 4 lg + lr / 4, dims 16 dt + 4 (lr % 4) + 0..3
        const int t = 4 * lg + (lr >> 2);
#pragma unroll
        for (int d2 = 0; d2 < NDT / 2; ++d2) {
          u32x2 vr[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int col = 16 * (2 * d2 + e) + 4 * (lr & 3);
            vr[e] = ds_read_tr16_raw(vslot + t * D + 8 * ((col >> 3) ^ vswz(t)) + (col & 7));
          }
          vv[d2] = u32x4{vr[0][0], vr[0][1], vr[1][0], vr[1][1]};
        }
      }
      lds_wait_all(vv);
#pragma unroll
      for (int d2 = 0; d2 < NDT / 2; ++d2)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const u32x2 va = {vv[d2][2 * e], vv[d2][2 * e + 1]};
          ot[2 * d2 + e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
              __builtin_bit_cast(s16x4, va), __builtin_bit_cast(s16x4, pb), ot[2 * d2 + e], 0, 0, 0);
        }
    }

    // ---- combine the 4 key rows of the wave (same reference per head) ----
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    // ---- combine the 4 waves: lane (lr < G, lg) holds dims 16 dt + 4 lg + i of head lr ----
    if (lr < G) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        *reinterpret_cast<f32x4*>(&s_acc[w][lr][16 * dt + 4 * lg]) = ot[dt];
      if (lg == 0) {
        s_m[w][lr] = l_run > 0.f ? m_run : -INFINITY;
        s_l[w][lr] = l_run;
      }
    }
    __syncthreads();
    const bool single = (n_parts == 1);
    for (int idx = tid; idx < G * D; idx += 256) {
      const int hh = idx / D, d = idx - (idx / D) * D;
      float M = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, s_m[ww][hh]);
      float L = 0.f, Acc = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float f = (s_m[ww][hh] == -INFINITY) ? 0.f : fast_exp2(s_m[ww][hh] - M);
        L += s_l[ww][hh] * f;
        Acc += s_acc[ww][hh][d] * f;
      }
      const int head = h0 + hh;
      if (single) {
        o[((int64_t)r * H_q + head) * D + d] = (uint16_t)f32_to_bf16_bits(L > 0.f ? Acc / L : 0.f);
      } else {
        float* wp = ws + (((int64_t)r * H_q + head) * max_parts + part) * (D + 2);
        wp[2 + d] = Acc;
        if (d == 0) {
          wp[0] = M;
          wp[1] = L;
        }
      }
    }
    __syncthreads();  // LDS is reused by the next item
  }
}

// ============================================================================
// Merge of the partition partials: o = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
// grid B * H_q, D threads. Requests with one partition were written directly;
// an empty context gives zeros.
// ============================================================================
template <typename T>
__global__ void k_paged_merge(T* __restrict__ o, const int32_t* __restrict__ ctx, int max_blocks,
                              int H_q, int D, int part_blocks, int max_parts,
                              const float* __restrict__ ws) {
  const int rh = blockIdx.x;
  const int r = rh / H_q;
  const int n_parts = n_parts_of(ctx[r], max_blocks, part_blocks, max_parts);
  if (n_parts == 1) return;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float out = 0.f;
    if (n_parts > 1) {
      const float* wp = ws + (int64_t)rh * max_parts * (D + 2);
      float M = -INFINITY;
      for (int p = 0; p < n_parts; ++p) M = fmaxf(M, wp[p * (D + 2)]);
      float L = 0.f, A = 0.f;
      for (int p = 0; p < n_parts; ++p) {
        const float f = (wp[p * (D + 2)] == -INFINITY) ? 0.f : fast_exp2(wp[p * (D + 2)] - M);
        L += wp[p * (D + 2) + 1] * f;
        A += wp[p * (D + 2) + 2 + d] * f;
      }
      out = L > 0.f ? A / L : 0.f;
    }
    io<T>::st(o, (int64_t)rh * D + d, out);
  }
}

// ============================================================================
// Simple paged attention (VALU), any dtype, decode or causal prefill: one wave
// per (query row, head). Each lane runs an online softmax over keys
// lane, lane+64, ...; lanes are merged by log-sum-exp through LDS. Used for
// fp32 I/O.
// ============================================================================
template <int D, typename T>
__global__ __launch_bounds__(64) void k_paged_attn_simple(
    const T* __restrict__ q, T* __restrict__ o, const T* __restrict__ k_pool,
    const T* __restrict__ v_pool, int64_t n_blocks, const int32_t* __restrict__ bt,
    int max_blocks, const int32_t* __restrict__ ctx, const int32_t* __restrict__ cu_q, int H_q,
    int H_kv, float scale_log2) {
  const int i = blockIdx.x, h = blockIdx.y, r = blockIdx.z;
  const int q0 = cu_q ? cu_q[r] : r;
  const int ql = cu_q ? cu_q[r + 1] - q0 : 1;
  if (i >= ql) return;
  const int row = q0 + i;
  const int n_keys = min(ctx[r] - ql + i + 1, max_blocks * kBlock);
  const int g = h / (H_q / H_kv);
  const int lane = threadIdx.x;
  __shared__ float sq[D];
  __shared__ float sacc[64][D + 1];
  __shared__ float sm[64], sl[64];
  for (int d = lane; d < D; d += 64) sq[d] = io<T>::ld(q, ((int64_t)row * H_q + h) * D + d);
  __syncthreads();
  float m = -INFINITY, lsum = 0.f;
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  const int32_t* btr = bt + (int64_t)r * max_blocks;
  for (int p = lane; p < n_keys; p += 64) {
    const int32_t blk = btr[p >> 4];
    if (blk < 0 || blk >= n_blocks) continue;  // defensive: invalid ids are skipped
    const int64_t base = (((int64_t)blk * H_kv + g) * kBlock + (p & 15)) * D;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) s = __builtin_fmaf(sq[d], io<T>::ld(k_pool, base + d), s);
    s *= scale_log2;
    const float mn = fmaxf(m, s);
    const float corr = fast_exp2(m - mn);
    const float pw = fast_exp2(s - mn);
    lsum = lsum * corr + pw;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(pw, io<T>::ld(v_pool, base + d), acc[d] * corr);
    m = mn;
  }
  sm[lane] = m;
  sl[lane] = lsum;
#pragma unroll
  for (int d = 0; d < D; ++d) sacc[lane][d] = acc[d];
  __syncthreads();
  float M = -INFINITY;
  for (int j = 0; j < 64; ++j) M = fmaxf(M, sm[j]);
  for (int d = lane; d < D; d += 64) {
    float L = 0.f, A = 0.f;
    if (n_keys > 0) {
      for (int j = 0; j < 64; ++j) {
        const float f = (sm[j] == -INFINITY) ? 0.f : fast_exp2(sm[j] - M);
        L += sl[j] * f;
        A += sacc[j][d] * f;
      }
    }
    io<T>::st(o, ((int64_t)row * H_q + h) * D + d, n_keys > 0 ? A / L : 0.f);
  }
}

template <int D, typename T>
static hipError_t launch_simple(const void* q, void* o, const void* k_pool, const void* v_pool,
                                int64_t n_blocks, const int32_t* bt, int max_blocks,
                                const int32_t* ctx, const int32_t* cu_q, int max_q_len, int B,
                                int H_q, int H_kv, float scale_log2, hipStream_t s) {
  dim3 grid((unsigned)max_q_len, (unsigned)H_q, (unsigned)B);
  hipLaunchKernelGGL((k_paged_attn_simple<D, T>), grid, dim3(64), 0, s, (const T*)q, (T*)o,
                     (const T*)k_pool, (const T*)v_pool, n_blocks, bt, max_blocks, ctx, cu_q, H_q,
                     H_kv, scale_log2);
  return hipGetLastError();
}

hipError_t launch_paged_simple_f32(const void* q, void* o, const void* k_pool, const void* v_pool,
                                   int64_t n_blocks, const int32_t* bt, int max_blocks,
                                   const int32_t* ctx, const int32_t* cu_q, int max_q_len, int B,
                                   int H_q, int H_kv, int D, float scale, hipStream_t s) {
  const float sl2 = scale * kLog2e;
  if (D == 128)
    return launch_simple<128, float>(q, o, k_pool, v_pool, n_blocks, bt, max_blocks, ctx, cu_q,
                                     max_q_len, B, H_q, H_kv, sl2, s);
  return launch_simple<64, float>(q, o, k_pool, v_pool, n_blocks, bt, max_blocks, ctx, cu_q,
                                  max_q_len, B, H_q, H_kv, sl2, s);
}

hipError_t launch_decode_plan(const int32_t* ctx, int max_context, int B, int H_q, int H_kv, int D,
                              int max_blocks, void* workspace, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  const DecodePlan plan = decode_plan(max_context, (int64_t)B * H_kv);
  int32_t* cu_parts = reinterpret_cast<int32_t*>(
      (char*)workspace + decode_partials_bytes(B, H_q, D, plan.max_parts));
  hipLaunchKernelGGL(k_decode_plan, dim3(1), dim3(1024), 0, s, ctx, B, max_blocks,
                     plan.part_blocks, plan.max_parts, cu_parts);
  return hipGetLastError();
}

hipError_t launch_paged_decode(const void* q, void* o, const void* k_pool, const void* v_pool,
                               int64_t n_blocks, const int32_t* bt, int max_blocks,
                               const int32_t* ctx, int max_context,
                               int B, int H_q, int H_kv, int D, float scale, void* workspace,
                               bool bf16, hipStream_t s, bool plan_ready) {
  if (B <= 0) return hipSuccess;
  const float sl2 = scale * kLog2e;
  if (!bf16) {
    if (D == 128)
      return launch_simple<128, float>(q, o, k_pool, v_pool, n_blocks, bt, max_blocks, ctx, nullptr, 1, B,
                                       H_q, H_kv, sl2, s);
    return launch_simple<64, float>(q, o, k_pool, v_pool, n_blocks, bt, max_blocks, ctx, nullptr, 1, B, H_q,
                                    H_kv, sl2, s);
  }
  const DecodePlan plan = decode_plan(max_context, (int64_t)B * H_kv);
  const int G = H_q / H_kv;
  float* ws = (float*)workspace;
  int32_t* cu_parts = reinterpret_cast<int32_t*>(
      (char*)workspace + decode_partials_bytes(B, H_q, D, plan.max_parts));
  hipError_t e = hipSuccess;
  if (!plan_ready) {
    e = launch_decode_plan(ctx, max_context, B, H_q, H_kv, D, max_blocks, workspace, s);
    if (e != hipSuccess) return e;
  }
  // enough workers to fill the chip a few times over; each walks items with stride gridDim.x
  const long bound = (long)B * plan.max_parts;
  unsigned workers = (unsigned)(bound < 2048 ? bound : 2048);
  if (workers > 8) workers &= ~7u;  // a multiple of the 8 XCDs (see the kernel)
  dim3 grid(workers * (unsigned)H_kv), block(256);
#define HY_PD(DD, GG)                                                                         \
  do {                                                                                        \
    constexpr size_t lds = decode_lds_bytes<DD>();                                            \
    static bool lds_set = false; /* the attribute is per device function; set once */         \
    if (!lds_set) {                                                                           \
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_paged_decode_bf16<DD, GG>),    \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);          \
      if (e != hipSuccess) return e;                                                          \
      lds_set = true;                                                                         \
    }                                                                                         \
    hipLaunchKernelGGL((k_paged_decode_bf16<DD, GG>), grid, block, lds, s, (const uint16_t*)q, \
                       (uint16_t*)o, (const uint16_t*)k_pool, (const uint16_t*)v_pool, n_blocks, \
                       bt, max_blocks, ctx, B, H_q, H_kv, sl2, plan.part_blocks, plan.max_parts, \
                       ws, cu_parts);                                                         \
  } while (0)
#define HY_PD_G(DD)                   \
  switch (G) {                        \
    case 1: HY_PD(DD, 1); break;      \
    case 2: HY_PD(DD, 2); break;      \
    case 4: HY_PD(DD, 4); break;      \
    case 8: HY_PD(DD, 8); break;      \
    default: return hipErrorInvalidValue; \
  }
  if (D == 128) {
    HY_PD_G(128)
  } else {
    HY_PD_G(64)
  }
#undef HY_PD_G
#undef HY_PD
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // partials of multi-partition requests are merged; empty contexts get zeros
  hipLaunchKernelGGL(k_paged_merge<uint16_t>, dim3((unsigned)(B * H_q)), dim3(D), 0, s,
                     (uint16_t*)o, ctx, max_blocks, H_q, D, plan.part_blocks, plan.max_parts, ws);
  return hipGetLastError();
}

}  // namespace hy
