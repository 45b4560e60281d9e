// Causal prefill attention over a paged KV cache of 16-token blocks for
// gfx950, bf16 I/O (MFMA, FlashAttention-style). fp32 I/O takes the VALU
// kernel in k_paged.hip.
//
// Method (page "推理框架适配Hybrid Model：KV Cache管理与算子调度实战", "P2"):
//   §2.1  KV is cut into fixed 16-token blocks mapped through a per-request
//         page (block) table.
//   §2.3  prefill is a FlashAttention-class kernel: softmax attention of each
//         new token over the request's cached tokens and the new ones before it.
// Layout: pool [n_blocks][H_kv][16][D]; logical token p of request r lives in
// block bt[r][p / 16] at offset p % 16; query head h reads KV head
// h / (H_q / H_kv). Softmax is evaluated in base 2 on scores pre-multiplied by
// scale * log2(e), with a running reference subtracted (fp32 throughout).
#include <math.h>

#include <algorithm>

#include "hy_common.hpp"
#include "hy_kernels.hpp"

namespace hy {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSum = 65536.f;     // bound on a lane's p-sum before the reference moves
constexpr float kMinusHuge = -0x1p100f;    // finite stand-in for -inf as a softmax reference
constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;  // bf16 pair (1, 1)

template <bool B> struct BoolTag { static constexpr bool value = B; };
// 16-row tiles per wave: three (48 rows) amortise each K/V stage, its barrier
// and its LDS reads over 1.5x the MFMA work of two, and still fit two waves
// per SIMD (256 VGPRs); four need a whole SIMD per wave and run slower
constexpr int kPrefillNR = 3;

// ============================================================================
// Causal prefill, bf16 (MFMA, FlashAttention-style). 1-D grid over (query
// tile, H_kv, B), 4 waves. A workgroup takes QT = 64 NR / G query positions
// of one request for all G query heads sharing KV head g (64 NR rows), so
// every K/V tile staged in LDS serves G heads. Wave w owns 16 NR rows (NR
// tiles of 16).
//
// K and V reach LDS through direct global-to-LDS loads (global_load_lds:
// no registers hold the data in flight) in 32-key stages (two 16-token
// blocks), kept in a ring of 4 stage buffers: stage st + 3 is requested
// while stage st is used, so three stages of loads are in flight behind the
// computation. Each lane's 16-byte load is aimed so that the tiles land
// XOR-swizzled per row (the K score reads and the V transposing reads are
// free of bank conflicts). Per stage:
//   S^T = K Q^T   (two 16-key tiles; the key order inside each tile is
//                  permuted so that a lane ends up with 8 consecutive keys of
//                  its row, i.e. directly the B operand below)
//   online softmax over the lane's row (see the stage body)
//   O^T += V^T P^T (A = V^T fragment via transposing LDS reads, B = P^T
//                  from registers)
// Computing O^T rather than O keeps the softmax row, the score column and the
// output column on the same lane, so rescaling needs no data movement.
//
// PERSIST = true: the same work items walked by a grid of at most one
// workgroup per CU (the hybrid step's form beside a decode on a second
// stream, which then keeps room on every CU), with a workgroup barrier before
// each item's first stage requests.
// ============================================================================
template <int D>
__host__ __device__ __forceinline__ int pf_kswz(int row) {  // chunk XOR of a K row of a stage
  if constexpr (D == 128) return (row & 3) | ((row >> 1) & 12);
  else return ((row >> 1) & 1) | ((row >> 2) & 6);
}
template <int D>
__host__ __device__ __forceinline__ int pf_vswz(int row) {  // chunk XOR of a V row of a stage (even)
  if constexpr (D == 128) return ((row & 3) << 1) | (row & 8);
  else return (row & 2) | (((row >> 3) & 1) << 2);
}

// All transposing reads of a stage's V operand as one opaque block: D / 16
// fragments, each two reads 4 rows apart, fragment i from LDS byte address
// a[i]. Opaque, so the compiler does not drain the global-to-LDS loads in
// flight before it (it would before its own transposing reads); it also does
// not see the block's register writes, so the leading s_nop provides the wait
// states that an MFMA issued just before the block needs when it still reads
// a register the block overwrites (the compiler inserts them for its own LDS
// loads). The caller waits (lds_wait_all) before using the fragments.
template <int D> __device__ __forceinline__ void tr_block(const uint32_t (&a)[D / 16], u32x4 (&vf)[D / 16]);
template <> __device__ __forceinline__ void tr_block<128>(const uint32_t (&a)[8], u32x4 (&vf)[8]) {
  u32x2 r[16];
  asm volatile(
      "s_nop 7\n"
      "ds_read_b64_tr_b16 %0, %16\n ds_read_b64_tr_b16 %1, %16 offset:1024\n"
      "ds_read_b64_tr_b16 %2, %17\n ds_read_b64_tr_b16 %3, %17 offset:1024\n"
      "ds_read_b64_tr_b16 %4, %18\n ds_read_b64_tr_b16 %5, %18 offset:1024\n"
      "ds_read_b64_tr_b16 %6, %19\n ds_read_b64_tr_b16 %7, %19 offset:1024\n"
      "ds_read_b64_tr_b16 %8, %20\n ds_read_b64_tr_b16 %9, %20 offset:1024\n"
      "ds_read_b64_tr_b16 %10, %21\n ds_read_b64_tr_b16 %11, %21 offset:1024\n"
      "ds_read_b64_tr_b16 %12, %22\n ds_read_b64_tr_b16 %13, %22 offset:1024\n"
      "ds_read_b64_tr_b16 %14, %23\n ds_read_b64_tr_b16 %15, %23 offset:1024"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]),
        "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]));
#pragma unroll
  for (int i = 0; i < 8; ++i) vf[i] = u32x4{r[2 * i][0], r[2 * i][1], r[2 * i + 1][0], r[2 * i + 1][1]};
}
template <> __device__ __forceinline__ void tr_block<64>(const uint32_t (&a)[4], u32x4 (&vf)[4]) {
  u32x2 r[8];
  asm volatile(
      "s_nop 7\n"
      "ds_read_b64_tr_b16 %0, %8\n ds_read_b64_tr_b16 %1, %8 offset:512\n"
      "ds_read_b64_tr_b16 %2, %9\n ds_read_b64_tr_b16 %3, %9 offset:512\n"
      "ds_read_b64_tr_b16 %4, %10\n ds_read_b64_tr_b16 %5, %10 offset:512\n"
      "ds_read_b64_tr_b16 %6, %11\n ds_read_b64_tr_b16 %7, %11 offset:512"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
#pragma unroll
  for (int i = 0; i < 4; ++i) vf[i] = u32x4{r[2 * i][0], r[2 * i][1], r[2 * i + 1][0], r[2 * i + 1][1]};
}

template <int D, int G, int NR, bool PERSIST>
__global__ __launch_bounds__(256, 2) void k_paged_prefill_bf16(
    const uint16_t* __restrict__ q, uint16_t* __restrict__ o, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, int64_t n_blocks, const int32_t* __restrict__ bt,
    int max_blocks, const int32_t* __restrict__ ctx, const int32_t* __restrict__ cu_q, int H_q,
    int H_kv, float scale_log2, int n_qt, int n_req) {
  constexpr int ROWS = 64 * NR; // rows (query position, head) per workgroup: 4 waves x 16 NR
  constexpr int QT = ROWS / G;  // query positions per workgroup
  constexpr int KS = D / 32;    // k steps over the head dim
  constexpr int NDT = D / 16;   // 16-wide head-dim tiles of O^T
  constexpr int KT = 32;        // keys per stage
  constexpr int NB = 4;         // stage buffers in the ring
  constexpr int CPR = D / 8;    // 16-byte chunks per row
  constexpr int RPI = 64 / CPR; // rows covered by one wave-wide 16-byte load
  constexpr int IPB = 16 / RPI; // such loads per 16-token block
  __shared__ __align__(16) uint16_t Ks[NB][KT * D];
  __shared__ __align__(16) uint16_t Vs[NB][KT * D];

  // 1-D grid in XCD-major order. Workgroup ids go round-robin over the 8
  // XCDs, so XCD x runs ids x, x + 8, ...; its j-th one takes (request, KV
  // head) pair 8 (j / n_qt) + x and query tile n_qt - 1 - j % n_qt. Each XCD
  // thus works through its pairs one after another, all query tiles of a
  // pair together, heaviest (longest causal span) first: the tiles in flight
  // on an XCD stream the same pair's keys, which its L2 then holds, and the
  // shortest tiles fill the tail. Ids past the last pair exit at once.
  // PERSIST: the same ids, walked by a smaller grid (see the end).
  const int n_gr = H_kv * n_req;
  auto item = [&](const int id) {
  const int xcd = id & 7, jx = id >> 3;
  const int pslot = jx / n_qt;
  const int pair = pslot * 8 + xcd;
  if (pair >= n_gr) return;
  const int qtile = n_qt - 1 - (jx - pslot * n_qt);
  const int g = pair % H_kv, r = pair / H_kv;
  const int q0 = cu_q[r], ql = cu_q[r + 1] - q0;
  const int i0 = qtile * QT;
  if (i0 >= ql) return;
  const int c = min(ctx[r], max_blocks * kBlock);
  const int base_pos = c - ql;  // position of this request's first query
  if (base_pos < 0 || n_blocks <= 0) return;  // more queries than context: invalid input
  const int kend = min(c, base_pos + i0 + QT);
  const int n_st = (kend + KT - 1) / KT;
  const int pos_lo = base_pos + i0;  // smallest query position of the workgroup
  const int32_t* btr = bt + (int64_t)r * max_blocks;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;

  // ---- rows of this lane: tile rt covers wave rows 16 rt .. 16 rt + 15 ----
  int row_pos[NR];   // query position inside the request (may be >= ql: padding)
  int row_head[NR];
  u32x4 qf[NR][KS];
#pragma unroll
  for (int rt = 0; rt < NR; ++rt) {
    const int R = w * 16 * NR + 16 * rt + lr;
    row_head[rt] = R / QT;
    row_pos[rt] = i0 + R % QT;
    const bool ok = row_pos[rt] < ql;
    const uint16_t* qp = q + ((int64_t)(q0 + row_pos[rt]) * H_q + g * G + row_head[rt]) * D + 8 * lg;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[rt][s] = ok ? *reinterpret_cast<const u32x4*>(qp + 32 * s) : u32x4{0u, 0u, 0u, 0u};
  }

  f32x4 ot[NDT][NR];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int rt = 0; rt < NR; ++rt) ot[dt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // m_run: the row's softmax reference in the scaled (log2) domain, starting
  // at a finite stand-in for -inf so that p = 2^(s - m) is +inf for any real
  // score (forcing the first exact pass) and 0 for a masked one (never NaN).
  // l_run: this lane's share of the row's sum of p.
  float m_run[NR], l_run[NR];
#pragma unroll
  for (int rt = 0; rt < NR; ++rt) {
    m_run[rt] = kMinusHuge;
    l_run[rt] = 0.f;
  }

  // ---- staging: wave w moves tensor (w & 1: K, V) of block (w >> 1) of
  // each stage, IPB wave-wide 16-byte loads straight into LDS. The block id
  // is wave-uniform (a scalar load, fetched one stage ahead of its use).
  // Lane l of load i fills row 16 b + RPI i + l / CPR, chunk position
  // l % CPR, so it fetches the logical chunk that the row's XOR maps there.
  const int w_s = __builtin_amdgcn_readfirstlane(w);
  const int sb = w_s >> 1;          // block of the stage this wave moves
  const bool sv = (w_s & 1) != 0;   // V (else K)
  const uint16_t* pool = sv ? v_pool : k_pool;
  auto block_of = [&](int st) -> int32_t {  // raw table entry, validated at use
    const int key = st * KT + kBlock * sb;
    return (st < n_st && key < c) ? btr[key >> 4] : -1;
  };
  auto issue_stage = [&](int st, int32_t blk) {
    if (blk < 0 || blk >= n_blocks) blk = 0;  // absent: any valid block, zeroed after landing
    const uint16_t* src = pool + ((int64_t)blk * H_kv + g) * kBlock * D;
    uint16_t* dst = (sv ? Vs[st % NB] : Ks[st % NB]) + kBlock * sb * D;
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
      const int tok = RPI * i + l / CPR;         // token within the block
      const int row = kBlock * sb + tok;         // row within the stage
      const int x = sv ? pf_vswz<D>(row) : pf_kswz<D>(row);
      __builtin_amdgcn_global_load_lds(src + tok * D + 8 * ((l % CPR) ^ x),
                                       (__attribute__((address_space(3))) void*)(dst + RPI * i * D),
                                       16, 0, 0);
    }
  };
  // rows of a landed stage that hold no valid key (past the context, or an
  // absent block) are cleared by the wave that moved them: V must be finite
  // there, as masked keys still meet it in P V with weight 0
  auto clear_invalid = [&](int st, int32_t blk) {
    const int key0 = st * KT + kBlock * sb;
    const int nvalid = (blk < 0 || blk >= n_blocks) ? 0 : min(kBlock, max(0, c - key0));
    if (nvalid == kBlock) return;
    uint16_t* dst = (sv ? Vs[st % NB] : Ks[st % NB]) + kBlock * sb * D;
    for (int e = l; e < kBlock * CPR; e += 64)
      if (e / CPR >= nvalid) *reinterpret_cast<u32x4*>(dst + 8 * e) = u32x4{0u, 0u, 0u, 0u};
  };

  // ---- scores S^T for the stage's 32 keys x this wave's rows ----
  // Lane (lr, lg) receives keys 8 lg + 4 u + i of row tile rt.
  auto scores = [&](const uint16_t* Kb, f32x4 (&sc)[2][NR]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int krow = 8 * (lr >> 2) + 4 * u + (lr & 3);
#pragma unroll
      for (int rt = 0; rt < NR; ++rt) sc[u][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const u32x4 kf =
            *reinterpret_cast<const u32x4*>(Kb + krow * D + 8 * ((4 * s + lg) ^ pf_kswz<D>(krow)));
#pragma unroll
        for (int rt = 0; rt < NR; ++rt) sc[u][rt] = mfma16x16x32(kf, qf[rt][s], sc[u][rt]);
      }
    }
  };

  // ---- online softmax pieces ----
  // p = 2^(s * scale_log2 - m_run), packed to bf16 pairs (the P^T operand);
  // returns the lane's sum of the rounded p, the values P V actually uses.
  auto probs = [&](const f32x4 (&sc)[2][NR], int rt, u32x4& pb) -> float {
    float x[8];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        x[4 * u + i] = fast_exp2(__builtin_fmaf(sc[u][rt][i], scale_log2, -m_run[rt]));
    float ps = 0.f;
#pragma unroll
    for (int p2 = 0; p2 < 4; ++p2) {
      pb[p2] = pack_bf16x2(x[2 * p2], x[2 * p2 + 1]);
      ps = dot2_bf16(pb[p2], kOnesBf16x2, ps);
    }
    return ps;
  };
  auto mask = [&](int key0, f32x4 (&sc)[2][NR]) {  // keys beyond each row's position
#pragma unroll
    for (int rt = 0; rt < NR; ++rt) {
      const int pos = base_pos + row_pos[rt];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (key0 + 8 * lg + 4 * u + i > pos) sc[u][rt][i] = -INFINITY;
    }
  };
  auto lane_max = [&](const f32x4 (&sc)[2][NR], int rt) -> float {
    return fmaxf(fmaxf(fmaxf(sc[0][rt][0], sc[0][rt][1]), fmaxf(sc[0][rt][2], sc[0][rt][3])),
                 fmaxf(fmaxf(sc[1][rt][0], sc[1][rt][1]), fmaxf(sc[1][rt][2], sc[1][rt][3])));
  };

  // ---- O^T += V^T P^T for the stage ----
  // V^T rows 16 dt + lr (head dims), keys 8 lg + 0..7: two transposing reads
  // per tile; source lane (lg, lr) addresses key row 8 lg + lr / 4 (+ 4),
  // head dims 16 dt + 4 (lr % 4) + 0..3 (rows + 4 share the row's XOR). The
  // reads go out as one opaque block (tr_block) after the softmax (with three
  // row tiles per wave, fragments requested before it would not fit the
  // registers); one explicit wait precedes the products.
  auto pv_load = [&](const uint16_t* Vb, u32x4 (&vf)[NDT]) {
    const int vrow = 8 * lg + (lr >> 2);
    uint32_t a[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int vcol = 16 * dt + 4 * (lr & 3);
      const uint16_t* vp = Vb + vrow * D + 8 * ((vcol >> 3) ^ pf_vswz<D>(vrow)) + (vcol & 7);
      a[dt] = static_cast<uint32_t>(
          reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const uint16_t*)vp));
    }
    tr_block<D>(a, vf);
  };
  auto pv_acc = [&](u32x4 (&vf)[NDT], const u32x4 (&pb)[NR]) {
    lds_wait_all(vf);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int rt = 0; rt < NR; ++rt) ot[dt][rt] = mfma16x16x32(vf[dt], pb[rt], ot[dt][rt]);
  };

  // One 32-key stage. Softmax: the common case needs no cross-lane work. p is
  // taken against the current reference m_run and each lane checks its own
  // sum; only when some lane's sum exceeds kRescaleSum (a score above the
  // reference by about log2(kRescaleSum), or the first keys of a row) does
  // the wave take the exact path: per row, the maximum over the stage's keys
  // across the four lanes holding it, a new reference, the rescale of the
  // row's partial sums and accumulators, and p again.
  auto compute = [&](auto diag, int st) {
    const uint16_t* Kb = Ks[st % NB];
    const uint16_t* Vb = Vs[st % NB];
    f32x4 sc[2][NR];
    u32x4 pb[NR];
    float ps[NR];
    // Wave priorities: two waves of different workgroups share each SIMD, so
    // while one runs its matrix products the other can run its softmax. The
    // softmax runs at priority 2 and the products at 1 (the ring waits and the
    // barrier at 0), so the SIMD's arbiter issues the VALU work of a wave in
    // its softmax ahead of the other wave's MFMAs, which then fill the matrix
    // pipe behind it: 5 % faster than equal priorities.
    __builtin_amdgcn_s_setprio(1);
    // LLVM's interleaving of LDS reads with MFMAs for small products
    // (iglp_opt 0) over the score phase: 4.5 % faster than its own schedule
    __builtin_amdgcn_iglp_opt(0);
    scores(Kb, sc);
    if constexpr (decltype(diag)::value) mask(st * KT, sc);
    __builtin_amdgcn_s_setprio(2);
    bool over = false;
#pragma unroll
    for (int rt = 0; rt < NR; ++rt) {
      ps[rt] = probs(sc, rt, pb[rt]);
      over |= !(ps[rt] <= kRescaleSum);  // also catches +inf
    }
    if (__builtin_amdgcn_ballot_w64(over)) {
      float corr[NR];
#pragma unroll
      for (int rt = 0; rt < NR; ++rt) {
        float mx = lane_max(sc, rt);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float ms = mx * scale_log2;  // -inf when every key of the stage is masked
        corr[rt] = 1.f;
        if (ms > m_run[rt]) {
          corr[rt] = fast_exp2(m_run[rt] - ms);  // 0 on the row's first real key
          l_run[rt] *= corr[rt];
          m_run[rt] = ms;
        }
        ps[rt] = probs(sc, rt, pb[rt]);
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int rt = 0; rt < NR; ++rt) {
          ot[dt][rt][0] *= corr[rt];
          ot[dt][rt][1] *= corr[rt];
          ot[dt][rt][2] *= corr[rt];
          ot[dt][rt][3] *= corr[rt];
        }
    }
#pragma unroll
    for (int rt = 0; rt < NR; ++rt) l_run[rt] += ps[rt];
    __builtin_amdgcn_s_setprio(1);
    u32x4 vf[NDT];
    pv_load(Vb, vf);
    pv_acc(vf, pb);
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- the stage ring ----
  // Each wave issues IPB loads per stage, and stages complete in order, so
  // waiting for stage st leaves the IPB loads of each later stage already
  // requested outstanding. Stage st + 3 goes into the buffer of stage st - 1,
  // which every wave finished reading before the barrier of stage st.
  int32_t blk_ring[NB];  // block ids of the stages in flight (wave-uniform)
  // the Q fragments land first, so no later wait for them can drain the ring
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  // a workgroup that walks several items: every wave is done with the previous
  // item's stage buffers before any wave requests this item's first stages
  if constexpr (PERSIST) __syncthreads();
#pragma unroll
  for (int i = 0; i < NB - 1; ++i) {
    blk_ring[i] = block_of(i);
    if (i < n_st) issue_stage(i, blk_ring[i]);
  }
  blk_ring[NB - 1] = block_of(NB - 1);
  auto stage = [&](auto diag, int st) {
    const int ahead = n_st - 1 - st;  // stages requested after this one: min(ahead, NB - 2)
    if (ahead >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * IPB));
    else if (ahead == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(IPB));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    const int32_t blk = blk_ring[0];
    if (st * KT + KT > c || blk < 0 || blk >= n_blocks) clear_invalid(st, blk);
    // workgroup barrier without the release fence of __syncthreads, which
    // would also drain the global-to-LDS loads still in flight: the stage's
    // own loads were waited for above and LDS writes are waited for here
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (st + NB - 1 < n_st) issue_stage(st + NB - 1, blk_ring[NB - 1]);
#pragma unroll
    for (int i = 0; i < NB - 1; ++i) blk_ring[i] = blk_ring[i + 1];
    compute(diag, st);
    // the block id after next is fetched after the compute: scalar loads
    // share the LDS counter, so earlier it would delay the LDS reads above
    blk_ring[NB - 1] = block_of(st + NB);
  };
  // stages whose keys all lie at or before the workgroup's first query
  // position need no causal mask
  const int n_plain = min(n_st, (pos_lo + 1) / KT);
  int st = 0;
  for (; st < n_plain; ++st) stage(BoolTag<false>{}, st);
  for (; st < n_st; ++st) stage(BoolTag<true>{}, st);

  // ---- normalise and store: lane holds O^T[d = 16 dt + 4 lg + i][row lr] ----
#pragma unroll
  for (int rt = 0; rt < NR; ++rt) {
    float L = l_run[rt];
    L += __shfl_xor(L, 16);
    L += __shfl_xor(L, 32);
    const float inv = 1.f / L;
    if (row_pos[rt] >= ql) continue;
    uint16_t* op = o + ((int64_t)(q0 + row_pos[rt]) * H_q + g * G + row_head[rt]) * D + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      u32x2 t;
      t[0] = pack_bf16x2(ot[dt][rt][0] * inv, ot[dt][rt][1] * inv);
      t[1] = pack_bf16x2(ot[dt][rt][2] * inv, ot[dt][rt][3] * inv);
      *reinterpret_cast<u32x2*>(op + 16 * dt) = t;
    }
  }
  };
  if constexpr (PERSIST) {
    // persistent: a grid of at most one workgroup per CU walks the ids with
    // stride gridDim.x (a multiple of 8, so each workgroup stays on its XCD's
    // ids, in the order above)
    const int n_ids = n_qt * 8 * ((n_gr + 7) / 8);
    for (int id = (int)blockIdx.x; id < n_ids; id += (int)gridDim.x) item(id);
  } else {
    item((int)blockIdx.x);
  }
}

hipError_t launch_paged_prefill(const void* q, void* o, const void* k_pool, const void* v_pool,
                                int64_t n_blocks, const int32_t* bt, int max_blocks,
                                const int32_t* ctx,
                                const int32_t* cu_q, int max_q_len, int B, int H_q, int H_kv,
                                int D, float scale, bool bf16, hipStream_t s, int grid_cap) {
  if (B <= 0 || max_q_len <= 0) return hipSuccess;
  const float sl2 = scale * kLog2e;
  if (bf16) {
    const int G = H_q / H_kv;
    // grid_cap > 0: at most that many workgroups (rounded down to a multiple of
    // 8), each walking several ids (the persistent form)
    const int cap = grid_cap > 0 ? std::max(8, grid_cap & ~7) : 0;
#define HY_PP(DD, GG)                                                                          \
  do {                                                                                         \
    constexpr int QT_ = 64 * kPrefillNR / GG;                                                  \
    const int n_qt = (max_q_len + QT_ - 1) / QT_;                                              \
    const int n_ids = n_qt * 8 * ((H_kv * B + 7) / 8);                                         \
    if (cap > 0 && cap < n_ids)                                                                \
      hipLaunchKernelGGL((k_paged_prefill_bf16<DD, GG, kPrefillNR, true>), dim3((unsigned)cap), \
                         dim3(256), 0, s, (const uint16_t*)q, (uint16_t*)o,                    \
                         (const uint16_t*)k_pool, (const uint16_t*)v_pool, n_blocks, bt,       \
                         max_blocks, ctx, cu_q, H_q, H_kv, sl2, n_qt, B);                      \
    else                                                                                       \
      hipLaunchKernelGGL((k_paged_prefill_bf16<DD, GG, kPrefillNR, false>), dim3((unsigned)n_ids), \
                         dim3(256), 0, s, (const uint16_t*)q, (uint16_t*)o,                    \
                         (const uint16_t*)k_pool, (const uint16_t*)v_pool, n_blocks, bt,       \
                         max_blocks, ctx, cu_q, H_q, H_kv, sl2, n_qt, B);                      \
  } while (0)
#define HY_PP_G(DD)                   \
  switch (G) {                        \
    case 1: HY_PP(DD, 1); break;      \
    case 2: HY_PP(DD, 2); break;      \
    case 4: HY_PP(DD, 4); break;      \
    case 8: HY_PP(DD, 8); break;      \
    default: return hipErrorInvalidValue; \
  }
    if (D == 128) {
      HY_PP_G(128)
    } else {
      HY_PP_G(64)
    }
#undef HY_PP_G
#undef HY_PP
    return hipGetLastError();
  }
  return launch_paged_simple_f32(q, o, k_pool, v_pool, n_blocks, bt, max_blocks, ctx, cu_q,
                                 max_q_len, B, H_q, H_kv, D, scale, s);
}

}  // namespace hy
