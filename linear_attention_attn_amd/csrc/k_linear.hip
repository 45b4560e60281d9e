// Linear-attention kernels for gfx950: state-slot zeroing, single-token
// decode, and chunked prefill.
//
// Method (page "推理框架适配Hybrid Model：KV Cache管理与算子调度实战", "P2"):
//   §2.1  per head a D x D state S; a token adds k (x) v, the output is q . S
//         (with the token already in S); decode costs O(D^2) per token.
//   §2.3  the state is zeroed when the request starts, accumulated by
//         prefill, read and updated by decode.
//   §2.4  chunked prefill carries S from chunk to chunk.
// Layout: states fp32 [layer][slot][H][D][D] with S[i][j] at i * D + j
// (row i = key dim, column j = value dim); q/k/v/o token-major [N][H][D].
#include <map>
#include <mutex>
#include <utility>

#include "hy_common.hpp"
#include "hy_kernels.hpp"


namespace hy {

constexpr float kLog2e = 1.4426950408889634f;  // exp(x) = 2^(x log2 e)

// ============================================================================
// Zeroing: S[l][slot] = 0 for every linear layer l and listed slot.
// grid (pieces, n, L); each block clears 64 KiB of one (layer, slot) region.
// ============================================================================
__global__ __launch_bounds__(256) void k_state_zero(float* __restrict__ pool, int n_slots,
                                                    int64_t slot_elems,
                                                    const int32_t* __restrict__ slots) {
  const int slot = slots[blockIdx.y];
  if (slot < 0 || slot >= n_slots) return;
  float* base = pool + ((int64_t)blockIdx.z * n_slots + slot) * slot_elems;
  const int64_t piece = 16384;  // floats per block
  const int64_t start = (int64_t)blockIdx.x * piece;
  const int64_t end = start + piece < slot_elems ? start + piece : slot_elems;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  for (int64_t i = start + 4 * threadIdx.x; i < end; i += 4 * 256)
    *reinterpret_cast<f32x4*>(base + i) = z;
}

hipError_t launch_state_zero(float* pool, int n_layers, int n_slots, int64_t slot_elems,
                             const int32_t* slots, int n, hipStream_t s) {
  if (n <= 0 || n_layers <= 0) return hipSuccess;
  const int64_t pieces = (slot_elems + 16383) / 16384;
  dim3 grid((unsigned)pieces, (unsigned)n, (unsigned)n_layers);
  hipLaunchKernelGGL(k_state_zero, grid, dim3(256), 0, s, pool, n_slots, slot_elems, slots);
  return hipGetLastError();
}

// ============================================================================
// Decode: one workgroup per (request, head) and column slice. S streams
// through registers once: with NCS slices of D / NCS value columns, each
// thread owns 4 adjacent columns of D / RG rows of its slice; it adds
// k[i] v[j], then accumulates q[i] S_new[i][j]. The per-thread partial
// outputs are summed over the row groups in LDS in a fixed order
// (deterministic); a slice's output columns need no other slice.
// Large batches take NCS = 4: four times the workgroups, each a quarter of a
// state, which evens out the last round over the CUs (3.7 % faster at 7 680
// (request, head) units). Smaller batches run k_linear_decode_p below over
// whole states (NCS = 1): the same per-thread arithmetic, so the same bits.
// XCD-major order: workgroup ids go round-robin over the 8 XCDs, and XCD x
// (ids x, x + 8, ...) takes the consecutive items x P .. x P + P - 1, so each
// XCD streams one contiguous eighth of the listed states. The grid has 8 P ids
// (P = ceil(items / 8)); ids past the last item exit.
// ============================================================================
template <int D, typename T, bool GATED, int NCS>
__global__ __launch_bounds__(256) void k_linear_decode(float* __restrict__ states, int n_slots,
                                                       const T* __restrict__ q,
                                                       const T* __restrict__ k,
                                                       const T* __restrict__ v, T* __restrict__ o,
                                                       const float* __restrict__ log_gamma,
                                                       const int32_t* __restrict__ slots, int H,
                                                       int n_units) {
  constexpr int DC = D / NCS;    // value columns of this workgroup
  constexpr int C4 = DC / 4;     // threads across a row (4 floats each)
  constexpr int RG = 256 / C4;   // row groups
  constexpr int RP = D / RG;     // rows per thread
  static_assert(RP >= 1 && RG * RP == D, "k_linear_decode: column split does not tile D");
  __shared__ float sq[D], sk[D], sv[DC];
  __shared__ float red[RG][DC];

  const int per = (int)gridDim.x >> 3;
  const int item = ((int)blockIdx.x & 7) * per + ((int)blockIdx.x >> 3);
  if (item >= n_units * NCS) return;
  const int unit = item / NCS;            // r * H + h
  const int col0 = (item - unit * NCS) * DC;
  const int r = unit / H;
  const int h = unit - r * H;
  const int slot = slots[r];
  if (slot < 0 || slot >= n_slots) return;
  float* S = states + ((int64_t)slot * H + h) * (int64_t)(D * D) + col0;
  const int64_t xo = (int64_t)unit * D;
  const int t = threadIdx.x;
  const int c4 = t % C4, rg = t / C4;

  f32x4 s[RP];
#pragma unroll
  for (int j = 0; j < RP; ++j)
    s[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (rg + RG * j) * D + 4 * c4));
  if (t < D) {
    sq[t] = io<T>::ld(q, xo + t);
    sk[t] = io<T>::ld(k, xo + t);
  }
  if (t < DC) sv[t] = io<T>::ld(v, xo + col0 + t);
  __syncthreads();

  const f32x4 vv = {sv[4 * c4], sv[4 * c4 + 1], sv[4 * c4 + 2], sv[4 * c4 + 3]};
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float gamma = 1.f;
  if constexpr (GATED) gamma = fast_exp2(log_gamma[unit] * kLog2e);
#pragma unroll
  for (int j = 0; j < RP; ++j) {
    const int row = rg + RG * j;
    const float kr = sk[row], qr = sq[row];
    f32x4 x = s[j];
    if constexpr (GATED) x *= gamma;  // S <- gamma S + k (x) v
    x[0] = __builtin_fmaf(kr, vv[0], x[0]);
    x[1] = __builtin_fmaf(kr, vv[1], x[1]);
    x[2] = __builtin_fmaf(kr, vv[2], x[2]);
    x[3] = __builtin_fmaf(kr, vv[3], x[3]);
    acc[0] = __builtin_fmaf(qr, x[0], acc[0]);
    acc[1] = __builtin_fmaf(qr, x[1], acc[1]);
    acc[2] = __builtin_fmaf(qr, x[2], acc[2]);
    acc[3] = __builtin_fmaf(qr, x[3], acc[3]);
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(S + row * D + 4 * c4));
  }
  red[rg][4 * c4 + 0] = acc[0];
  red[rg][4 * c4 + 1] = acc[1];
  red[rg][4 * c4 + 2] = acc[2];
  red[rg][4 * c4 + 3] = acc[3];
  __syncthreads();
  if (t < DC) {
    float sum = 0.f;
#pragma unroll
    for (int g = 0; g < RG; ++g) sum += red[g][t];
    io<T>::st(o, xo + col0 + t, sum);
  }
}

// Persistent form of the decode: a fixed grid of workgroups, each walking the
// items item0, item0 + G, item0 + 2 G, ... (G = grid size). The state loads of
// the next item are requested before the current item's state is stored, so
// every wave keeps one item's reads in flight while it computes and writes the
// other; the next item's slot id is read one item earlier still, so the
// dependent slot -> state address never stalls a wave. On the 64-request,
// 32-head batch (134 MB of state, evicted from the caches before each step)
// this takes a step from 54.5 to 51.3 us; a plain read-modify-write stream of
// the same bytes runs at 47.6-50 us. Same arithmetic, per element, as
// k_linear_decode.
template <int D, typename T, bool GATED, int NCS, int NT>
__global__ __launch_bounds__(NT) void k_linear_decode_p(float* __restrict__ states, int n_slots,
                                                         const T* __restrict__ q,
                                                         const T* __restrict__ k,
                                                         const T* __restrict__ v, T* __restrict__ o,
                                                         const float* __restrict__ log_gamma,
                                                         const int32_t* __restrict__ slots, int H,
                                                         int n_units) {
  constexpr int DC = D / NCS;
  constexpr int C4 = DC / 4;
  constexpr int RG = NT / C4;
  constexpr int RP = D / RG;
  static_assert(RP >= 1 && RG * RP == D, "k_linear_decode_p: column split does not tile D");
  __shared__ float sq[D], sk[D], sv[DC];
  __shared__ float red[RG][DC];
  const int n_items = n_units * NCS;
  const int G = (int)gridDim.x;
  const int t = threadIdx.x;
  const int c4 = t % C4, rg = t / C4;

  // Per item: its slot is read one item ahead of its state, and its state,
  // q, k and v are requested one item ahead of their use, so no wait on a
  // slot id or an input vector stalls the item in hand.
  auto slot_of = [&](int item) -> int {
    return item < n_items ? slots[(item / NCS) / H] : -1;
  };
  auto state_of = [&](int item, int slot) -> float* {
    if (item >= n_items || slot < 0 || slot >= n_slots) return nullptr;
    const int unit = item / NCS;
    return states + ((int64_t)slot * H + (unit - (unit / H) * H)) * (int64_t)(D * D) +
           (item - unit * NCS) * DC;
  };
  auto load = [&](const float* S, f32x4 (&s)[RP]) {
#pragma unroll
    for (int j = 0; j < RP; ++j)
      s[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (rg + RG * j) * D + 4 * c4));
  };
  struct Vec { float q, k, v; };
  auto load_qkv = [&](int item) -> Vec {
    Vec x = {0.f, 0.f, 0.f};
    if (item >= n_items) return x;
    const int unit = item / NCS;
    const int64_t xo = (int64_t)unit * D;
    if (t < D) {
      x.q = io<T>::ld(q, xo + t);
      x.k = io<T>::ld(k, xo + t);
    }
    if (t < DC) x.v = io<T>::ld(v, xo + (item - unit * NCS) * DC + t);
    return x;
  };
  auto stage_qkv = [&](const Vec& x) {
    if (t < D) {
      sq[t] = x.q;
      sk[t] = x.k;
    }
    if (t < DC) sv[t] = x.v;
  };

  int item = blockIdx.x;
  if (item >= n_items) return;
  f32x4 sa[RP], sb[RP];
  float* Sa = state_of(item, slot_of(item));
  if (Sa) load(Sa, sa);
  stage_qkv(load_qkv(item));
  int slot_n = slot_of(item + G);  // slot of the next item
  float* Sb = nullptr;
  // item `it` (state in cur at Scur); its successor nit = it + G goes to nxt
  auto step = [&](f32x4 (&cur)[RP], float* Scur, f32x4 (&nxt)[RP], float*& Snxt, int it) {
    const int nit = it + G;
    Snxt = state_of(nit, slot_n);
    if (Snxt) load(Snxt, nxt);
    const Vec xn = load_qkv(nit);
    slot_n = slot_of(nit + G);
    __syncthreads();  // q, k, v of this item staged
    const int unit = it / NCS;
    const int col0 = (it - unit * NCS) * DC;
    const f32x4 vv = {sv[4 * c4], sv[4 * c4 + 1], sv[4 * c4 + 2], sv[4 * c4 + 3]};
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float gamma = 1.f;
    if constexpr (GATED) gamma = fast_exp2(log_gamma[unit] * kLog2e);
    if (Scur) {
#pragma unroll
      for (int j = 0; j < RP; ++j) {
        const int row = rg + RG * j;
        const float kr = sk[row], qr = sq[row];
        f32x4 x = cur[j];
        if constexpr (GATED) x *= gamma;  // S <- gamma S + k (x) v
        x[0] = __builtin_fmaf(kr, vv[0], x[0]);
        x[1] = __builtin_fmaf(kr, vv[1], x[1]);
        x[2] = __builtin_fmaf(kr, vv[2], x[2]);
        x[3] = __builtin_fmaf(kr, vv[3], x[3]);
        acc[0] = __builtin_fmaf(qr, x[0], acc[0]);
        acc[1] = __builtin_fmaf(qr, x[1], acc[1]);
        acc[2] = __builtin_fmaf(qr, x[2], acc[2]);
        acc[3] = __builtin_fmaf(qr, x[3], acc[3]);
        __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(Scur + row * D + 4 * c4));
      }
    }
    red[rg][4 * c4 + 0] = acc[0];
    red[rg][4 * c4 + 1] = acc[1];
    red[rg][4 * c4 + 2] = acc[2];
    red[rg][4 * c4 + 3] = acc[3];
    __syncthreads();  // partial outputs written; q, k, v no longer read
    if (Scur && t < DC) {
      float sum = 0.f;
#pragma unroll
      for (int g = 0; g < RG; ++g) sum += red[g][t];
      io<T>::st(o, (int64_t)unit * D + col0 + t, sum);
    }
    stage_qkv(xn);
    return nit;
  };
  for (;;) {
    item = step(sa, Sa, sb, Sb, item);
    if (item >= n_items) break;
    item = step(sb, Sb, sa, Sa, item);
    if (item >= n_items) break;
  }
}

// (request, head) units from which the decode splits each state over 4 workgroups
constexpr int64_t kDecodeSplitUnits = 4096;

// Workgroups of the persistent decode: two per CU at its register use
constexpr int kDecodePersistGrid = 512;

hipError_t launch_linear_decode(float* layer_states, int n_slots, const void* q, const void* k,
                                const void* v, void* o, const float* log_gamma,
                                const int32_t* slots, int B, int H, int D, bool bf16,
                                hipStream_t s) {
  if (B <= 0) return hipSuccess;
  const int64_t units = (int64_t)B * H;
  const bool split = units >= kDecodeSplitUnits;
  const dim3 block(256);
  // large batches: one-shot workgroups over quarter states; smaller ones: the
  // persistent form over whole states (each workgroup walks several)
  const dim3 grid((unsigned)(split ? 8 * ((4 * units + 7) / 8)
                                   : (units < kDecodePersistGrid ? units : kDecodePersistGrid)));
#define HY_DEC(DD, TT, GG)                                                                        \
  do {                                                                                            \
    if (split)                                                                                    \
      hipLaunchKernelGGL((k_linear_decode<DD, TT, GG, 4>), grid, block, 0, s, layer_states,       \
                         n_slots, (const TT*)q, (const TT*)k, (const TT*)v, (TT*)o, log_gamma,    \
                         slots, H, B * H);                                                        \
    else                                                                                          \
      hipLaunchKernelGGL((k_linear_decode_p<DD, TT, GG, 1, 256>), grid, block, 0, s,              \
                         layer_states, n_slots, (const TT*)q, (const TT*)k, (const TT*)v, (TT*)o, \
                         log_gamma, slots, H, B * H);                                             \
  } while (0)
#define HY_DEC_G(DD, TT)         \
  do {                           \
    if (log_gamma) {             \
      HY_DEC(DD, TT, true);      \
    } else {                     \
      HY_DEC(DD, TT, false);     \
    }                            \
  } while (0)
  if (D == 128) {
    if (bf16) HY_DEC_G(128, uint16_t); else HY_DEC_G(128, float);
  } else {
    if (bf16) HY_DEC_G(64, uint16_t); else HY_DEC_G(64, float);
  }
#undef HY_DEC_G
#undef HY_DEC
  return hipGetLastError();
}

// ============================================================================
// Chunked prefill, fp32 I/O (VALU). One workgroup per (request, head); S and
// the chunk's causal scores P live in LDS. Per chunk of n <= C tokens:
//   P[a][b] = q_a . k_b for b <= a (else 0)
//   o_a     = q_a . S + sum_b P[a][b] v_b
//   S      += sum_b k_b (x) v_b
// ============================================================================
//
// Gated variant (GATED): token a of the chunk brings log forget factor g_a;
// with L_a = g_0 + ... + g_a over the chunk (kept in LDS in log2 units),
//   P[a][b] *= exp(L_a - L_b),  o_a = exp(L_a) q_a . S + sum_b P[a][b] v_b,
//   S = exp(L_last) S + sum_b exp(L_last - L_b) k_b (x) v_b.
template <int D, bool GATED>
__global__ __launch_bounds__(256) void k_linear_prefill_f32(float* __restrict__ states,
                                                            int n_slots,
                                                            const float* __restrict__ q,
                                                            const float* __restrict__ k,
                                                            const float* __restrict__ v,
                                                            float* __restrict__ o,
                                                            const float* __restrict__ log_gamma,
                                                            const int32_t* __restrict__ cu,
                                                            const int32_t* __restrict__ slots,
                                                            int H, int C) {
  extern __shared__ __align__(16) float lds_f[];
  float* Ss = lds_f;          // D * D
  float* P = lds_f + D * D;   // C * C
  float* Lc = P + C * C;      // C: L_a in log2 units (gated)
  float* Wc = Lc + C;         // C: exp(L_last - L_b) (gated)
  const int unit = blockIdx.x;
  const int r = unit / H, h = unit - (unit / H) * H;
  const int tok0 = cu[r], T = cu[r + 1] - tok0;
  const int slot = slots[r];
  if (T <= 0 || slot < 0 || slot >= n_slots) return;
  float* S = states + ((int64_t)slot * H + h) * (int64_t)(D * D);
  const int64_t ldx = (int64_t)H * D;
  const float* qb = q + (int64_t)tok0 * ldx + (int64_t)h * D;
  const float* kb = k + (int64_t)tok0 * ldx + (int64_t)h * D;
  const float* vb = v + (int64_t)tok0 * ldx + (int64_t)h * D;
  float* ob = o + (int64_t)tok0 * ldx + (int64_t)h * D;
  const int t = threadIdx.x;
  for (int i = t; i < D * D; i += 256) Ss[i] = S[i];
  __syncthreads();
  for (int c0 = 0; c0 < T; c0 += C) {
    const int n = (T - c0 < C) ? (T - c0) : C;
    if constexpr (GATED) {
      if (t == 0) {  // running sum in token order
        float run = 0.f;
        for (int a = 0; a < n; ++a) {
          run += log_gamma[(int64_t)(tok0 + c0 + a) * H + h] * kLog2e;
          Lc[a] = run;
        }
      }
      __syncthreads();
      for (int b = t; b < n; b += 256) Wc[b] = fast_exp2(Lc[n - 1] - Lc[b]);
    }
    for (int idx = t; idx < n * n; idx += 256) {
      const int a = idx / n, b = idx - (idx / n) * n;
      float s = 0.f;
      if (b <= a) {
        const float* qa = qb + (int64_t)(c0 + a) * ldx;
        const float* kk = kb + (int64_t)(c0 + b) * ldx;
        for (int i = 0; i < D; ++i) s = __builtin_fmaf(qa[i], kk[i], s);
        if constexpr (GATED) s *= fast_exp2(Lc[a] - Lc[b]);
      }
      P[a * C + b] = s;
    }
    __syncthreads();
    for (int idx = t; idx < n * D; idx += 256) {
      const int a = idx / D, j = idx % D;
      const float* qa = qb + (int64_t)(c0 + a) * ldx;
      float acc = 0.f;
      for (int i = 0; i < D; ++i) acc = __builtin_fmaf(qa[i], Ss[i * D + j], acc);
      if constexpr (GATED) acc *= fast_exp2(Lc[a]);
      for (int b = 0; b <= a; ++b) acc = __builtin_fmaf(P[a * C + b], vb[(int64_t)(c0 + b) * ldx + j], acc);
      ob[(int64_t)(c0 + a) * ldx + j] = acc;
    }
    __syncthreads();
    const float decay = GATED ? fast_exp2(Lc[n - 1]) : 1.f;
    for (int idx = t; idx < D * D; idx += 256) {
      const int i = idx / D, j = idx % D;
      float acc = 0.f;
      for (int b = 0; b < n; ++b) {
        float kw = kb[(int64_t)(c0 + b) * ldx + i];
        if constexpr (GATED) kw *= Wc[b];
        acc = __builtin_fmaf(kw, vb[(int64_t)(c0 + b) * ldx + j], acc);
      }
      if constexpr (GATED)
        Ss[idx] = __builtin_fmaf(decay, Ss[idx], acc);
      else
        Ss[idx] += acc;
    }
    __syncthreads();
  }
  for (int i = t; i < D * D; i += 256) S[i] = Ss[i];
}

// ============================================================================
// Chunked prefill, bf16 I/O, MFMA (v_mfma_f32_16x16x32_bf16).
//
// One workgroup (4 waves) per (request, head). Wave w owns the value columns
// [w*D/4, (w+1)*D/4) of the state, kept in fp32 accumulator registers for the
// whole request. Per chunk, K and V are staged in LDS (64 KiB at C = 128, so
// two workgroups share a CU and hide each other's staging), and the query
// rows are taken two 16-row tiles at a time (both see the same key blocks,
// so each K or V fragment read from LDS serves two tiles). For its value
// columns each wave computes
//   O_c^T = S^T Q_c^T   (S split into bf16 hi + lo: two MFMAs, fp32-faithful)
//         + V_c^T tril(Q_c K_c^T)^T   (scores in fp32, split hi + lo likewise)
//   S    += K_c^T V_c   (accumulated straight into the fp32 state registers)
// O^T rather than O puts four consecutive value columns of one query row in
// a lane, so outputs leave as 8-byte stores. Token-contiguous operands (V
// columns, K^T rows) come from row-major tiles through the transposing LDS
// read. Index permutations keep the other operands contiguous reads:
//  * state rows: accumulator tile t, row m holds key dim
//      pi(t, m) = 32*(t/2) + 8*(m/4) + 4*(t%2) + m%4
//    so that tiles 2s and 2s+1 together give each lane the 8 consecutive key
//    dims 32s + 8*(l/16) + 0..7 that its Q fragment holds;
//  * score tiles: P^T = K Q^T over 32 keys as two 16-row tiles whose row m
//    is key 8*(m/4) + 4u + m%4 (u = tile), so each lane ends up with the 8
//    consecutive keys 8*(l/16) + 0..7 of one query row, i.e. directly the B
//    operand of V^T P^T.
// LDS rows hold D elements with their 16-byte chunks XOR-swizzled per row,
// chosen so that each access pattern (Q and K fragment reads over 16 rows,
// transposing reads over 4-8 rows, 16-byte staging writes) spreads over all
// banks.
// ============================================================================
template <int D>
struct PrefillCfg {
  static constexpr int NW = 4;
  static constexpr int DVW = D / NW;   // value columns per wave
  static constexpr int NDV = DVW / 16; // 16-wide value tiles per wave
  static constexpr int NDK = D / 16;   // 16-row key-dim tiles of the state
  static constexpr int KS = D / 32;    // 32-wide k steps over the head dim
  static constexpr int CPR = D / 8;    // 16-byte chunks per row
};

__device__ __forceinline__ int state_row(int t, int m) {
  return 32 * (t >> 1) + 8 * (m >> 2) + 4 * (t & 1) + (m & 3);
}

// chunk XORs of the staged tiles (rows relative to the tile)
template <int D>
__device__ __forceinline__ int qswz(int row) {
  if constexpr (D == 128) return row & 15;
  else return (row >> 1) & 7;
}
template <int D>
__device__ __forceinline__ int kswz(int row) {
  if constexpr (D == 128) return ((row >> 3) & 3) | ((row & 3) << 2);
  else return ((row >> 3) & 3) | (((row >> 1) & 1) << 2);
}
template <int D>
__device__ __forceinline__ int vswz(int row) {
  if constexpr (D == 128) return ((row & 3) << 1) | (row & 8);
  else return (row & 2) | (((row >> 3) & 1) << 2);
}
// element offset of (row, col) in a tile with chunk XOR x
template <int D>
__device__ __forceinline__ int swz_off(int row, int col, int x) {
  return row * D + 8 * ((col >> 3) ^ x) + (col & 7);
}
__device__ __forceinline__ void split8(const float* x, u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t h, l;
    split_bf16x2(x[2 * p], x[2 * p + 1], h, l);
    hi[p] = h;
    lo[p] = l;
  }
}

// Raw transposing read of the same operand (see ds_read_tr16_raw): for loops
// that keep global-to-LDS loads in flight. Wait with lds_wait_all before use.
template <int D, bool IS_K>
__device__ __forceinline__ u32x4 tr_swz_raw(const uint16_t* tile, int col_src) {
  const int l = threadIdx.x & 63;
  const int row = 8 * (l >> 4) + ((l & 15) >> 2);
  const uint16_t* p = tile + swz_off<D>(row, col_src, IS_K ? kswz<D>(row) : vswz<D>(row));
  const u32x2 a = ds_read_tr16_raw(p);
  const u32x2 b = ds_read_tr16_raw(p + 4 * D);
  return u32x4{a[0], a[1], b[0], b[1]};
}

// Token blocks of the bf16 prefill: 32 tokens, i.e. one pair of 16-row MFMA
// tiles. The state is brought up to date after every block, so a block's
// output needs the causal scores of the block itself only.
constexpr int kLinBlock = 32;
// LDS ring of token blocks (K, V and Q tiles of 32 x D each, + gates)
constexpr int kLinRing = 3;

template <int D, bool GATED>
struct LinRing {
  static constexpr int TILE = kLinBlock * D;              // elements of one tile
  static constexpr int GATE = GATED ? 4 * 64 * 2 : 0;     // 4 waves x 64 fp32 (as bf16 units)
  static constexpr int SLOT = 3 * TILE + GATE;            // elements (uint16) per slot
  static constexpr int CPR = D / 8;                       // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;                    // rows per 1 KiB load instruction
  static constexpr int IPT = kLinBlock / RPI;             // load instructions per tile
  static constexpr int IPB = 3 * IPT / 4;                 // tile loads per wave per block
  static constexpr int VMB = IPB + (GATED ? 1 : 0);       // vector-memory loads per wave per block
  static_assert(3 * IPT % 4 == 0, "tile loads split evenly over 4 waves");
};

template <int D>
size_t prefill_bf16_lds_bytes(int /*C*/, bool gated) {
  return gated ? (size_t)kLinRing * LinRing<D, true>::SLOT * 2
               : (size_t)kLinRing * LinRing<D, false>::SLOT * 2;
}

// Chunked prefill, streaming form. One workgroup (4 waves) per (request,
// head); wave w keeps value columns [w D/4, (w+1) D/4) of the fp32 state in
// accumulator registers for the whole request. The request's tokens pass in
// 32-token blocks; K, V and Q of block b move from HBM straight into a
// 3-slot LDS ring (global_load_lds, no registers hold the data in flight),
// requested two blocks ahead of their use, with each lane's 16-byte load
// aimed so that the tiles land XOR-swizzled per row. Per block, each wave
// computes for its value columns
//   O_b^T = S^T Q_b^T               (S split into bf16 hi + lo: fp32-faithful)
//         + V_b^T tril(Q_b K_b^T)^T (scores in fp32, split hi + lo likewise)
//   S    += K_b^T V_b
// which is the chunk form of P2 §2.4 with 32-token chunks: any chunking gives
// the same sums, so the caller's chunk size only fixes the reference it is
// compared against. One barrier per block, with no release fence: output
// stores stay in flight across it; transposing reads are issued as opaque
// instructions so that the compiler does not drain the ring's loads before
// them.
// Gated variant (GATED): the block's 32 log forget factors travel with the
// tiles (each wave loads its own copy); a 32-lane scan gives L_a = g_0 + ..
// + g_a over the block, and
//   O_b^T = exp(L_a) S^T q_a + V_b^T (tril(Q_b K_b^T) * exp(L_a - L_c))^T
//   S     = exp(L_last) S + K_b^T diag(exp(L_last - L_c)) V_b
// with the weighted V split hi + lo.
template <int D, bool GATED>
__global__ __launch_bounds__(256, 2) void k_linear_prefill_bf16(
    float* __restrict__ states, int n_slots, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
    const float* __restrict__ log_gamma, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ slots, int H, int /*C*/) {
  using Cfg = PrefillCfg<D>;
  using R = LinRing<D, GATED>;
  constexpr int NDV = Cfg::NDV, NDK = Cfg::NDK, KS = Cfg::KS, CPR = R::CPR, RPI = R::RPI;
  constexpr int TILE = R::TILE, IPT = R::IPT, IPB = R::IPB, VMB = R::VMB;
  extern __shared__ __align__(16) uint16_t lds_h[];

  const int unit = blockIdx.x;
  const int r = unit / H, h = unit - (unit / H) * H;
  const int tok0 = cu[r], T = cu[r + 1] - tok0;
  const int slot = slots[r];
  if (T <= 0 || slot < 0 || slot >= n_slots) return;
  const int nb = (T + kLinBlock - 1) / kLinBlock;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
  const int dv0 = w * Cfg::DVW;
  float* S = states + ((int64_t)slot * H + h) * (int64_t)(D * D);
  const int64_t ldx = (int64_t)H * D;
  const uint16_t* qb = q + (int64_t)tok0 * ldx + (int64_t)h * D;
  const uint16_t* kb = k + (int64_t)tok0 * ldx + (int64_t)h * D;
  const uint16_t* vb = v + (int64_t)tok0 * ldx + (int64_t)h * D;
  uint16_t* ob = o + (int64_t)tok0 * ldx + (int64_t)h * D;

  // ---- block loads: the block's 3 IPT pieces (K pieces, then V, then Q; RPI
  // rows each) go round-robin over the waves, so load i of wave w is piece
  // 4 i + w: its tensor, 4 i / IPT, is known at compile time and its rows are
  // piece (4 i) % IPT + w of that tensor. A lane's source address is the
  // block's first token row (a wave-uniform 64-bit base) plus a small row
  // offset (24-bit multiply; the launcher checks that H D fits). Rows past
  // the request's end load its last token (finite data; V rows are cleared
  // before use, K and Q rows only meet masked scores or unstored outputs).
  static_assert(IPT % 4 == 0, "pieces of a tensor split evenly over 4 waves");
  auto piece_row = [&](int i) { return ((4 * i) % IPT + w) * RPI + l / CPR; };
  auto piece_swz = [&](int i, int row) {
    const int tensor = 4 * i / IPT;
    return tensor == 0 ? kswz<D>(row) : (tensor == 1 ? vswz<D>(row) : qswz<D>(row));
  };
  auto issue = [&](int b, int sl) {
    uint16_t* base = lds_h + sl * R::SLOT;
    const int64_t blk = (int64_t)(kLinBlock * b) * ldx;
    const int last = T - 1 - kLinBlock * b;  // last valid row of the block
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
      const int tensor = 4 * i / IPT;
      const int row = piece_row(i);
      const int rr = min(row, last);
      const uint32_t off = (uint32_t)__mul24(rr, (int)ldx) + 8 * ((l % CPR) ^ piece_swz(i, row));
      const uint16_t* src = (tensor == 0 ? kb : (tensor == 1 ? vb : qb)) + blk + off;
      uint16_t* dst = base + tensor * TILE + ((4 * i) % IPT + w) * RPI * D;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
    }
    if constexpr (GATED) {  // this wave's copy of the block's forget factors (lanes 32..63 repeat)
      const int tok = min(kLinBlock * b + (l & 31), T - 1);
      const float* src = log_gamma + (int64_t)(tok0 + tok) * H + h;
      uint16_t* dst = base + 3 * TILE + w * 128;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 4, 0, 0);
    }
  };
  // V rows past the request's end, among this wave's pieces, become zeros
  auto clear_tail = [&](int sl, int n) {
    uint16_t* base = lds_h + sl * R::SLOT;
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
      const int row = piece_row(i);
      if (4 * i / IPT == 1 && row >= n)
        *reinterpret_cast<u32x4*>(base + TILE + ((4 * i) % IPT + w) * RPI * D + 8 * l) =
            u32x4{0u, 0u, 0u, 0u};
    }
  };

  f32x4 Sacc[NDK][NDV];
#pragma unroll
  for (int t = 0; t < NDK; ++t)
#pragma unroll
    for (int n = 0; n < NDV; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Sacc[t][n][i] = S[(int64_t)state_row(t, 4 * lg + i) * D + dv0 + 16 * n + lr];

#pragma unroll
  for (int i = 0; i < kLinRing - 1; ++i)
    if (i < nb) issue(i, i);

  for (int b = 0; b < nb; ++b) {
    const int sl = b % kLinRing;
    const int n = min(kLinBlock, T - kLinBlock * b);
    // this wave's loads of block b have landed (block b + 1's may still fly)
    if (b + 1 < nb) __builtin_amdgcn_s_waitcnt(vmcnt_imm(VMB));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    if (n < kLinBlock) clear_tail(sl, n);
    lds_barrier();  // block b visible to all waves; block b - 1's slot is free
    if (b + kLinRing - 1 < nb) issue(b + kLinRing - 1, (b + kLinRing - 1) % kLinRing);

    const uint16_t* Kt = lds_h + sl * R::SLOT;
    const uint16_t* Vt = Kt + TILE;
    const uint16_t* Qt = Vt + TILE;

    // gated: L of the lane's query rows and keys, and of the block's last token
    float lrow[2] = {0.f, 0.f}, lkey[8], last = 0.f;
    if constexpr (GATED) {
      const float* gw = reinterpret_cast<const float*>(Qt + TILE) + w * 64;
      float x = ((l & 31) < n) ? gw[l & 31] * kLog2e : 0.f;
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) {
        const float y = __shfl_up(x, off, 32);
        if ((l & 31) >= off) x += y;
      }
      lrow[0] = __shfl(x, lr, 64);
      lrow[1] = __shfl(x, 16 + lr, 64);
#pragma unroll
      for (int e = 0; e < 8; ++e) lkey[e] = __shfl(x, 8 * lg + e, 64);
      last = __shfl(x, 31, 64);
    }

    // inter-block O^T = S^T Q^T (state before this block) and intra-block
    // scores P^T = K Q^T (two 16-key tiles), one 32-wide k step at a time so
    // each Q fragment serves both products; the fragments of step s + 1 are
    // requested before the products of step s
    f32x4 Ot[2][NDV];
    f32x4 pt[2][2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
      for (int nn = 0; nn < NDV; ++nn) Ot[t2][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 2; ++u) pt[t2][u] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    auto load_qk = [&](int s, u32x4 (&qf)[2], u32x4 (&kf)[2]) {
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const int row = 16 * t2 + lr;
        qf[t2] = *reinterpret_cast<const u32x4*>(Qt + swz_off<D>(row, 32 * s + 8 * lg, qswz<D>(row)));
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int krow = 8 * (lr >> 2) + 4 * u + (lr & 3);
        kf[u] = *reinterpret_cast<const u32x4*>(Kt + swz_off<D>(krow, 32 * s + 8 * lg, kswz<D>(krow)));
      }
    };
    u32x4 qf[2], kf[2];
    load_qk(0, qf, kf);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 qn[2], kn[2];
      if (s + 1 < KS) load_qk(s + 1, qn, kn);
#pragma unroll
      for (int nn = 0; nn < NDV; ++nn) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = Sacc[2 * s][nn][i];
          x[4 + i] = Sacc[2 * s + 1][nn][i];
        }
        u32x4 shi, slo;
        split8(x, shi, slo);
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          Ot[t2][nn] = mfma16x16x32(shi, qf[t2], Ot[t2][nn]);
          Ot[t2][nn] = mfma16x16x32(slo, qf[t2], Ot[t2][nn]);
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) pt[t2][u] = mfma16x16x32(kf[u], qf[t2], pt[t2][u]);
      if (s + 1 < KS) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          qf[i] = qn[i];
          kf[i] = kn[i];
        }
      }
    }
    if constexpr (GATED) {
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const float f = fast_exp2(lrow[t2]);
#pragma unroll
        for (int nn = 0; nn < NDV; ++nn) Ot[t2][nn] *= f;
      }
    }

    u32x4 phi[2], plo[2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int row = 16 * t2 + lr;
      float pv[8];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 8 * lg + 4 * u + i;
          float p = pt[t2][u][i];
          if constexpr (GATED) p *= fast_exp2(lrow[t2] - lkey[4 * u + i]);
          pv[4 * u + i] = (key <= row) ? p : 0.f;
        }
      split8(pv, phi[t2], plo[t2]);
    }

    // O^T += V^T P^T
    u32x4 vf[NDV];
#pragma unroll
    for (int nn = 0; nn < NDV; ++nn) vf[nn] = tr_swz_raw<D, false>(Vt, dv0 + 16 * nn + 4 * (lr & 3));
    lds_wait_all(vf);
#pragma unroll
    for (int nn = 0; nn < NDV; ++nn)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        Ot[t2][nn] = mfma16x16x32(vf[nn], phi[t2], Ot[t2][nn]);
        Ot[t2][nn] = mfma16x16x32(vf[nn], plo[t2], Ot[t2][nn]);
      }

    // lane holds O^T[value col 16 nn + 4 lg + i][query row lr] of each tile
    if constexpr (NDV == 2) {
      // lanes lg and lg ^ 1 (16 apart) swap a half so that each holds 8
      // consecutive columns of its row: lg even columns 4 lg .. 4 lg + 7,
      // lg odd columns 16 + 4 (lg - 1) .. + 7; every row of the wave's slice
      // then leaves as four aligned 16-byte pieces, whole 64-byte segments
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const int row = 16 * t2 + lr;
        uint32_t a0 = pack_bf16x2(Ot[t2][0][0], Ot[t2][0][1]);
        uint32_t a1 = pack_bf16x2(Ot[t2][0][2], Ot[t2][0][3]);
        uint32_t b0 = pack_bf16x2(Ot[t2][1][0], Ot[t2][1][1]);
        uint32_t b1 = pack_bf16x2(Ot[t2][1][2], Ot[t2][1][3]);
        const bool even = (lg & 1) == 0;
        const uint32_t s0 = even ? b0 : a0, s1 = even ? b1 : a1;  // the half the partner keeps
        const uint32_t r0 = __shfl_xor(s0, 16), r1 = __shfl_xor(s1, 16);
        const u32x4 piece = even ? u32x4{a0, a1, r0, r1} : u32x4{r0, r1, b0, b1};
        const int col = even ? 4 * lg : 16 + 4 * (lg - 1);
        if (row < n) {
          uint16_t* orow = ob + (int64_t)(kLinBlock * b) * ldx + (uint32_t)(row * (int)ldx + dv0 + col);
          *reinterpret_cast<u32x4*>(orow) = piece;
        }
      }
    } else {
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const int row = 16 * t2 + lr;
        if (row < n) {
          uint16_t* orow = ob + (int64_t)(kLinBlock * b) * ldx + (uint32_t)(row * (int)ldx + dv0 + 4 * lg);
#pragma unroll
          for (int nn = 0; nn < NDV; ++nn) {
            u32x2 t4;
            t4[0] = pack_bf16x2(Ot[t2][nn][0], Ot[t2][nn][1]);
            t4[1] = pack_bf16x2(Ot[t2][nn][2], Ot[t2][nn][3]);
            *reinterpret_cast<u32x2*>(orow + 16 * nn) = t4;
          }
        }
      }
    }

    // state update: S += K_b^T V_b (gated: S = exp(L_last) S + K_b^T W V_b)
    u32x4 kt[NDK];
#pragma unroll
    for (int t = 0; t < NDK; ++t)  // A operand: K^T rows pi(t, m) = columns of the K tile
      kt[t] = tr_swz_raw<D, true>(Kt, 32 * (t >> 1) + 8 * (lr & 3) + 4 * (t & 1));
    lds_wait_all(kt);
    if constexpr (GATED) {
      const float decay = fast_exp2(last);
#pragma unroll
      for (int t = 0; t < NDK; ++t)
#pragma unroll
        for (int nn = 0; nn < NDV; ++nn) Sacc[t][nn] *= decay;
      // the lane's V operand holds tokens 8 (l / 16) + 0..7 of the block
      float wt[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) wt[e] = fast_exp2(last - lkey[e]);
#pragma unroll
      for (int nn = 0; nn < NDV; ++nn) {
        float x[8];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          x[2 * p] = bf16_lo(vf[nn][p]) * wt[2 * p];
          x[2 * p + 1] = bf16_hi(vf[nn][p]) * wt[2 * p + 1];
        }
        u32x4 vhi, vlo;
        split8(x, vhi, vlo);
#pragma unroll
        for (int t = 0; t < NDK; ++t) {
          Sacc[t][nn] = mfma16x16x32(kt[t], vhi, Sacc[t][nn]);
          Sacc[t][nn] = mfma16x16x32(kt[t], vlo, Sacc[t][nn]);
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < NDK; ++t)
#pragma unroll
        for (int nn = 0; nn < NDV; ++nn) Sacc[t][nn] = mfma16x16x32(kt[t], vf[nn], Sacc[t][nn]);
    }
  }

#pragma unroll
  for (int t = 0; t < NDK; ++t)
#pragma unroll
    for (int n = 0; n < NDV; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S[(int64_t)state_row(t, 4 * lg + i) * D + dv0 + 16 * n + lr] = Sacc[t][n][i];
}

// ============================================================================
// Chunked prefill, bf16 I/O, D = 128, on v_mfma_f32_32x32x16_bf16.
//
// The same streaming form as k_linear_prefill_bf16 (same LDS ring of 32-token
// K, V and Q tiles, same loads, same per-block arithmetic), with every product
// on 32x32 tiles: wave w owns the 32 value columns v0 = 32 w .. v0 + 31 of the
// fp32 state, held as four 32x32 accumulator tiles (key dims 32 t .. 32 t + 31).
// Per block, per wave:
//   O^T = S^T Q^T             8 k steps of 16 key dims, S split hi + lo
//   P^T = K Q^T               the same 8 k steps (each Q fragment serves both)
//   O^T += V^T tril(P)^T      2 k steps of 16 keys, P split hi + lo
//   S  += K^T V               4 tiles x 2 k steps of 16 tokens
// Rows of every 32-row operand are permuted by perm32 (hy_common.hpp), so that the
// accumulator elements a lane holds are, per half-tile, eight consecutive
// indices: exactly the k operand the next product needs, with no data
// movement between lanes; the output then leaves as 16-byte pieces. The
// contractions' operands otherwise come straight from the row-major tiles
// (16-byte reads) or through transposing reads (K^T, V^T).
// ============================================================================

template <bool GATED>
__global__ __launch_bounds__(256, 2) void k_linear_prefill_m32(
    float* __restrict__ states, int n_slots, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
    const float* __restrict__ log_gamma, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ slots, int H) {
  constexpr int D = 128;
  using R = LinRing<D, GATED>;
  constexpr int CPR = R::CPR, RPI = R::RPI;
  constexpr int TILE = R::TILE, IPT = R::IPT, IPB = R::IPB, VMB = R::VMB;
  extern __shared__ __align__(16) uint16_t lds_h[];

  const int unit = blockIdx.x;
  const int r = unit / H, h = unit - (unit / H) * H;
  const int tok0 = cu[r], T = cu[r + 1] - tok0;
  const int slot = slots[r];
  if (T <= 0 || slot < 0 || slot >= n_slots) return;
  const int nb = (T + kLinBlock - 1) / kLinBlock;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int lc = l & 31, hl = l >> 5;        // MFMA column of the lane, its half
  const int gi = l & 15, gq = (l >> 4) & 1;  // place in its 16-lane group, the group's half-tile
  const int v0 = 32 * w;
  float* S = states + ((int64_t)slot * H + h) * (int64_t)(D * D);
  const int64_t ldx = (int64_t)H * D;
  const uint16_t* qb = q + (int64_t)tok0 * ldx + (int64_t)h * D;
  const uint16_t* kb = k + (int64_t)tok0 * ldx + (int64_t)h * D;
  const uint16_t* vb = v + (int64_t)tok0 * ldx + (int64_t)h * D;
  uint16_t* ob = o + (int64_t)tok0 * ldx + (int64_t)h * D;

  // ---- block loads (as k_linear_prefill_bf16) ----
  static_assert(IPT % 4 == 0, "pieces of a tensor split evenly over 4 waves");
  auto piece_row = [&](int i) { return ((4 * i) % IPT + w) * RPI + l / CPR; };
  auto piece_swz = [&](int i, int row) {
    const int tensor = 4 * i / IPT;
    return tensor == 0 ? kswz<D>(row) : (tensor == 1 ? vswz<D>(row) : qswz<D>(row));
  };
  auto issue = [&](int b, int sl) {
    uint16_t* base = lds_h + sl * R::SLOT;
    const int64_t blk = (int64_t)(kLinBlock * b) * ldx;
    const int last = T - 1 - kLinBlock * b;  // last valid row of the block
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
      const int tensor = 4 * i / IPT;
      const int row = piece_row(i);
      const int rr = min(row, last);
      const uint32_t off = (uint32_t)__mul24(rr, (int)ldx) + 8 * ((l % CPR) ^ piece_swz(i, row));
      const uint16_t* src = (tensor == 0 ? kb : (tensor == 1 ? vb : qb)) + blk + off;
      uint16_t* dst = base + tensor * TILE + ((4 * i) % IPT + w) * RPI * D;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
    }
    if constexpr (GATED) {  // this wave's copy of the block's forget factors (lanes 32..63 repeat)
      const int tok = min(kLinBlock * b + (l & 31), T - 1);
      const float* src = log_gamma + (int64_t)(tok0 + tok) * H + h;
      uint16_t* dst = base + 3 * TILE + w * 128;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 4, 0, 0);
    }
  };
  auto clear_tail = [&](int sl, int n) {  // V rows past the request's end become zeros
    uint16_t* base = lds_h + sl * R::SLOT;
#pragma unroll
    for (int i = 0; i < IPB; ++i) {
      const int row = piece_row(i);
      if (4 * i / IPT == 1 && row >= n)
        *reinterpret_cast<u32x4*>(base + TILE + ((4 * i) % IPT + w) * RPI * D + 8 * l) =
            u32x4{0u, 0u, 0u, 0u};
    }
  };

  // ---- transposing reads: for c = 0, 1 eight consecutive rows 16 c + 8 hl +
  // 0..7 of one column of a tile, the column being base + perm32(lc). The
  // lane's source address is row 16 c + 8 hl + gi / 4 (and 4 rows on, which
  // share its chunk XOR), 4-column piece base + 16 gq + {0, 8, 4, 12}[gi % 4]:
  // within each 16-lane group this hands lane gi the column
  // perm32(16 gq + gi). All four reads go out as one opaque block led by an
  // s_nop: an MFMA issued just before may still read registers the block
  // overwrites (the previous tile's fragments), and the compiler, which pads
  // its own LDS loads for that, does not see inside the block.
  auto tr8x2 = [&](const uint16_t* tile, int base, bool is_k, u32x4 (&f)[2]) {
    uint32_t a[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int row = 16 * c + 8 * hl + (gi >> 2);
      const int col = base + 16 * gq + 8 * (gi & 1) + 4 * ((gi >> 1) & 1);
      const uint16_t* p = tile + swz_off<D>(row, col, is_k ? kswz<D>(row) : vswz<D>(row));
      a[c] = static_cast<uint32_t>(
          reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const uint16_t*)p));
    }
    u32x2 r0, r1, r2, r3;
    asm volatile(
        "s_nop 7\n"
        "ds_read_b64_tr_b16 %0, %4\n ds_read_b64_tr_b16 %1, %4 offset:1024\n"
        "ds_read_b64_tr_b16 %2, %5\n ds_read_b64_tr_b16 %3, %5 offset:1024"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
        : "v"(a[0]), "v"(a[1]));
    f[0] = u32x4{r0[0], r0[1], r1[0], r1[1]};
    f[1] = u32x4{r2[0], r2[1], r3[0], r3[1]};
  };

  // state tiles: Sacc[t][i] = S[32 t + 16 (i >> 3) + 8 hl + (i & 7)][v0 + perm32(lc)]
  f32x16 Sacc[4];
  const int vcol = v0 + perm32(lc);
  {
    const float* Sin = S + (int64_t)(8 * hl) * D + vcol;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) Sacc[t][i] = Sin[(32 * t + 16 * (i >> 3) + (i & 7)) * D];
  }

#pragma unroll
  for (int i = 0; i < kLinRing - 1; ++i)
    if (i < nb) issue(i, i);

  for (int b = 0; b < nb; ++b) {
    const int sl = b % kLinRing;
    const int n = min(kLinBlock, T - kLinBlock * b);
    if (b + 1 < nb) __builtin_amdgcn_s_waitcnt(vmcnt_imm(VMB));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    if (n < kLinBlock) clear_tail(sl, n);
    lds_barrier();  // block b visible to all waves; block b - 1's slot is free
    if (b + kLinRing - 1 < nb) issue(b + kLinRing - 1, (b + kLinRing - 1) % kLinRing);

    const uint16_t* Kt = lds_h + sl * R::SLOT;
    const uint16_t* Vt = Kt + TILE;
    const uint16_t* Qt = Vt + TILE;

    // gated: L of the lane's query row lc and of its keys 16 a + 8 hl + e
    float lrow = 0.f, lkey[2][8], last = 0.f;
    if constexpr (GATED) {
      const float* gw = reinterpret_cast<const float*>(Qt + TILE) + w * 64;
      float x = ((l & 31) < n) ? gw[l & 31] * kLog2e : 0.f;
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) {
        const float y = __shfl_up(x, off, 32);
        if ((l & 31) >= off) x += y;
      }
      lrow = __shfl(x, lc, 64);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int e = 0; e < 8; ++e) lkey[a][e] = __shfl(x, 16 * a + 8 * hl + e, 64);
      last = __shfl(x, 31, 64);
    }

    // O^T = S^T Q^T and P^T = K Q^T, one 16-wide k step s at a time: the Q
    // fragment (query row lc, dims 16 s + 8 hl .. + 7) serves both; the
    // fragments of step s + 1 are requested before the products of step s
    f32x16 Ot, Pt;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      Ot[i] = 0.f;
      Pt[i] = 0.f;
    }
    const int krow = perm32(lc);
    auto load_qk = [&](int s, u32x4& qf, u32x4& kf) {
      qf = *reinterpret_cast<const u32x4*>(Qt + swz_off<D>(lc, 16 * s + 8 * hl, qswz<D>(lc)));
      kf = *reinterpret_cast<const u32x4*>(Kt + swz_off<D>(krow, 16 * s + 8 * hl, kswz<D>(krow)));
    };
    u32x4 qf, kf;
    load_qk(0, qf, kf);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 qn, kn;
      if (s + 1 < 8) load_qk(s + 1, qn, kn);
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = Sacc[s >> 1][8 * (s & 1) + e];
      u32x4 shi, slo;
      split8(x, shi, slo);
      Ot = mfma32x32x16(shi, qf, Ot);
      Ot = mfma32x32x16(slo, qf, Ot);
      Pt = mfma32x32x16(kf, qf, Pt);
      if (s + 1 < 8) {
        qf = qn;
        kf = kn;
      }
      // keep the scheduler from hoisting later steps' reads and splits (they
      // would hold many more registers than one step ahead needs)
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (GATED) Ot *= fast_exp2(lrow);

    // causal scores of query row lc: element i is key 16 (i >> 3) + 8 hl + (i & 7)
    u32x4 phi[2], plo[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = 16 * a + 8 * hl + e;
        float p = Pt[8 * a + e];
        if constexpr (GATED) p *= fast_exp2(lrow - lkey[a][e]);
        pv[e] = (key <= lc) ? p : 0.f;
      }
      split8(pv, phi[a], plo[a]);
    }

    // O^T += V^T P^T: V^T rows = value columns v0 + perm32(lc), keys 16 c + 8 hl + e
    u32x4 vt[2];
    tr8x2(Vt, v0, false, vt);
    lds_wait_all(vt);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      Ot = mfma32x32x16(vt[c], phi[c], Ot);
      Ot = mfma32x32x16(vt[c], plo[c], Ot);
    }

    // element i of Ot: value column v0 + 16 (i >> 3) + 8 hl + (i & 7) of query row lc
    if (lc < n) {
      uint16_t* orow = ob + (int64_t)(kLinBlock * b) * ldx + (uint32_t)(lc * (int)ldx + v0 + 8 * hl);
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        u32x4 piece;
#pragma unroll
        for (int p2 = 0; p2 < 4; ++p2) piece[p2] = pack_bf16x2(Ot[8 * a + 2 * p2], Ot[8 * a + 2 * p2 + 1]);
        *reinterpret_cast<u32x4*>(orow + 16 * a) = piece;
      }
    }

    // S += K^T V (gated: S = exp(L_last) S + K^T diag(exp(L_last - L_c)) V)
    u32x4 vw_hi[2], vw_lo[2];
    if constexpr (GATED) {
      const float decay = fast_exp2(last);
#pragma unroll
      for (int t = 0; t < 4; ++t) Sacc[t] *= decay;
      // vt[c] holds V of tokens 16 c + 8 hl + e
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float x[8];
#pragma unroll
        for (int p2 = 0; p2 < 4; ++p2) {
          x[2 * p2] = bf16_lo(vt[c][p2]) * fast_exp2(last - lkey[c][2 * p2]);
          x[2 * p2 + 1] = bf16_hi(vt[c][p2]) * fast_exp2(last - lkey[c][2 * p2 + 1]);
        }
        split8(x, vw_hi[c], vw_lo[c]);
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u32x4 kt[2];
      tr8x2(Kt, 32 * t, true, kt);
      lds_wait_all(kt);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        if constexpr (GATED) {
          Sacc[t] = mfma32x32x16(kt[c], vw_hi[c], Sacc[t]);
          Sacc[t] = mfma32x32x16(kt[c], vw_lo[c], Sacc[t]);
        } else {
          Sacc[t] = mfma32x32x16(kt[c], vt[c], Sacc[t]);
        }
      }
    }
  }

  // the state's addresses again (an opaque copy of the column keeps the
  // compiler from holding the load's 64 addresses across the whole loop)
  int vcol_out = vcol, hl_out = hl;
  asm volatile("" : "+v"(vcol_out), "+v"(hl_out));
  float* Sout = S + (int64_t)(8 * hl_out) * D + vcol_out;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) Sout[(32 * t + 16 * (i >> 3) + (i & 7)) * D] = Sacc[t][i];
}

size_t linear_prefill_bf16_lds_bytes(int D, int C, bool gated) {
  return D == 128 ? prefill_bf16_lds_bytes<128>(C, gated) : prefill_bf16_lds_bytes<64>(C, gated);
}

// Dynamic LDS above 64 KiB must be allowed per device function and device.
// The allowance is raised only when a launch needs more than it already
// grants: hipFuncSetAttribute on every launch costs host time that would
// show between short back-to-back launches.
template <typename K>
static hipError_t allow_lds(K kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, size_t> allowed;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const auto key = std::make_pair(reinterpret_cast<const void*>(kernel), dev);
  std::lock_guard<std::mutex> lk(mu);
  size_t& have = allowed[key];
  if (have >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(key.first, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) have = bytes;
  return e;
}

hipError_t device_cus(int* out) {
  static std::mutex mu;
  static std::map<int, int> cus;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cus.find(dev);
  if (it == cus.end()) {
    int n = 0;
    if ((e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
      return e;
    it = cus.emplace(dev, n).first;
  }
  *out = it->second;
  return hipSuccess;
}

hipError_t launch_linear_prefill(float* layer_states, int n_slots, const void* q, const void* k,
                                 const void* v, void* o, const float* log_gamma,
                                 const int32_t* cu, const int32_t* slots, int n_req, int H, int D,
                                 int chunk, bool bf16, hipStream_t s) {
  if (n_req <= 0) return hipSuccess;
  dim3 grid((unsigned)(n_req * H)), block(256);
  const bool gated = log_gamma != nullptr;
  hipError_t e;
  if (bf16) {
    // the block loads form a lane's row offset with a 24-bit multiply by H D
    if ((int64_t)H * D >= (1 << 23)) return hipErrorInvalidValue;
#define HY_LP(DD, GG)                                                                          \
  do {                                                                                         \
    const size_t lds = prefill_bf16_lds_bytes<DD>(chunk, GG);                                  \
    if ((e = allow_lds(k_linear_prefill_bf16<DD, GG>, lds)) != hipSuccess) return e;           \
    hipLaunchKernelGGL((k_linear_prefill_bf16<DD, GG>), grid, block, lds, s, layer_states,     \
                       n_slots, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,    \
                       (uint16_t*)o, log_gamma, cu, slots, H, chunk);                          \
  } while (0)
    int cus = 0;
    if ((e = device_cus(&cus)) != hipSuccess) return e;
    // One workgroup per CU: the 32x32-tile kernel (half the matrix instructions
    // lets one wave per SIMD keep pace with the loads). Two or more per CU: the
    // 16x16-tile kernel, whose co-resident waves overlap their phases as well.
    if (D == 128 && (int64_t)n_req * H <= cus) {
      const size_t lds = prefill_bf16_lds_bytes<128>(chunk, gated);
#define HY_LP32(GG)                                                                            \
  do {                                                                                         \
    if ((e = allow_lds(k_linear_prefill_m32<GG>, lds)) != hipSuccess) return e;                \
    hipLaunchKernelGGL((k_linear_prefill_m32<GG>), grid, block, lds, s, layer_states, n_slots, \
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,             \
                       (uint16_t*)o, log_gamma, cu, slots, H);                                 \
  } while (0)
      if (gated) HY_LP32(true); else HY_LP32(false);
#undef HY_LP32
    } else if (D == 128) {
      if (gated) HY_LP(128, true); else HY_LP(128, false);
    } else {
      if (gated) HY_LP(64, true); else HY_LP(64, false);
    }
#undef HY_LP
  } else {
    const size_t lds = (size_t)(D * D + chunk * chunk + (gated ? 2 * chunk : 0)) * sizeof(float);
#define HY_LPF(DD, GG)                                                                           \
  do {                                                                                           \
    if ((e = allow_lds(k_linear_prefill_f32<DD, GG>, lds)) != hipSuccess) return e;              \
    hipLaunchKernelGGL((k_linear_prefill_f32<DD, GG>), grid, block, lds, s, layer_states,        \
                       n_slots, (const float*)q, (const float*)k, (const float*)v, (float*)o,    \
                       log_gamma, cu, slots, H, chunk);                                          \
  } while (0)
    if (D == 128) {
      if (gated) HY_LPF(128, true); else HY_LPF(128, false);
    } else {
      if (gated) HY_LPF(64, true); else HY_LPF(64, false);
    }
#undef HY_LPF
  }
  return hipGetLastError();
}

}  // namespace hy
