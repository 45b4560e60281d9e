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
#include "hy_common.hpp"
#include "hy_kernels.hpp"

namespace hy {

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
// Decode: one workgroup per (request, head). S streams through registers once:
// each thread owns 4 adjacent columns of D/RG rows; it adds k[i] v[j], then
// accumulates q[i] S_new[i][j]. The per-thread partial outputs are summed over
// the row groups in LDS in a fixed order (deterministic).
// ============================================================================
template <int D, typename T>
__global__ __launch_bounds__(256) void k_linear_decode(float* __restrict__ states, int n_slots,
                                                       const T* __restrict__ q,
                                                       const T* __restrict__ k,
                                                       const T* __restrict__ v, T* __restrict__ o,
                                                       const int32_t* __restrict__ slots, int H) {
  constexpr int C4 = D / 4;      // threads across a row (4 floats each)
  constexpr int RG = 256 / C4;   // row groups
  constexpr int RP = D / RG;     // rows per thread
  __shared__ float sq[D], sk[D], sv[D];
  __shared__ float red[RG][D];

  const int unit = blockIdx.x;  // r * H + h
  const int r = unit / H;
  const int h = unit - r * H;
  const int slot = slots[r];
  if (slot < 0 || slot >= n_slots) return;
  float* S = states + ((int64_t)slot * H + h) * (int64_t)(D * D);
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
    sv[t] = io<T>::ld(v, xo + t);
  }
  __syncthreads();

  const f32x4 vv = {sv[4 * c4], sv[4 * c4 + 1], sv[4 * c4 + 2], sv[4 * c4 + 3]};
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < RP; ++j) {
    const int row = rg + RG * j;
    const float kr = sk[row], qr = sq[row];
    f32x4 x = s[j];
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
  if (t < D) {
    float sum = 0.f;
#pragma unroll
    for (int g = 0; g < RG; ++g) sum += red[g][t];
    io<T>::st(o, xo + t, sum);
  }
}

hipError_t launch_linear_decode(float* layer_states, int n_slots, const void* q, const void* k,
                                const void* v, void* o, const int32_t* slots, int B, int H, int D,
                                bool bf16, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  dim3 grid((unsigned)(B * H)), block(256);
#define HY_DEC(DD, TT)                                                                        \
  hipLaunchKernelGGL((k_linear_decode<DD, TT>), grid, block, 0, s, layer_states, n_slots,     \
                     (const TT*)q, (const TT*)k, (const TT*)v, (TT*)o, slots, H)
  if (D == 128) {
    if (bf16) HY_DEC(128, uint16_t); else HY_DEC(128, float);
  } else {
    if (bf16) HY_DEC(64, uint16_t); else HY_DEC(64, float);
  }
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
template <int D>
__global__ __launch_bounds__(256) void k_linear_prefill_f32(float* __restrict__ states,
                                                            int n_slots,
                                                            const float* __restrict__ q,
                                                            const float* __restrict__ k,
                                                            const float* __restrict__ v,
                                                            float* __restrict__ o,
                                                            const int32_t* __restrict__ cu,
                                                            const int32_t* __restrict__ slots,
                                                            int H, int C) {
  extern __shared__ __align__(16) float lds_f[];
  float* Ss = lds_f;          // D * D
  float* P = lds_f + D * D;   // C * C
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
    for (int idx = t; idx < n * n; idx += 256) {
      const int a = idx / n, b = idx - (idx / n) * n;
      float s = 0.f;
      if (b <= a) {
        const float* qa = qb + (int64_t)(c0 + a) * ldx;
        const float* kk = kb + (int64_t)(c0 + b) * ldx;
        for (int i = 0; i < D; ++i) s = __builtin_fmaf(qa[i], kk[i], s);
      }
      P[a * C + b] = s;
    }
    __syncthreads();
    for (int idx = t; idx < n * D; idx += 256) {
      const int a = idx / D, j = idx % D;
      const float* qa = qb + (int64_t)(c0 + a) * ldx;
      float acc = 0.f;
      for (int i = 0; i < D; ++i) acc = __builtin_fmaf(qa[i], Ss[i * D + j], acc);
      for (int b = 0; b <= a; ++b) acc = __builtin_fmaf(P[a * C + b], vb[(int64_t)(c0 + b) * ldx + j], acc);
      ob[(int64_t)(c0 + a) * ldx + j] = acc;
    }
    __syncthreads();
    for (int idx = t; idx < D * D; idx += 256) {
      const int i = idx / D, j = idx % D;
      float acc = 0.f;
      for (int b = 0; b < n; ++b)
        acc = __builtin_fmaf(kb[(int64_t)(c0 + b) * ldx + i], vb[(int64_t)(c0 + b) * ldx + j], acc);
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
// whole request. Per chunk, K and V are staged row-major in LDS (72 KiB at
// C = 128, so two workgroups share a CU and hide each other's staging); Q
// fragments come straight from global memory. Each wave computes, for its
// value columns:
//   O_c   = Q_c S  (S split into bf16 hi + lo, two MFMAs: fp32-faithful)
//         + tril(Q_c K_c^T) V_c  (scores in fp32, split hi + lo likewise)
//   S    += K_c^T V_c (accumulated straight into the fp32 state registers)
// Token-contiguous operands (K^T rows, V columns) are read from the
// row-major tiles with the transposing LDS read. Index permutations keep the
// other operands contiguous 16-byte reads:
//  * state rows: accumulator tile t, row m holds key dim
//      pi(t, m) = 32*(t/2) + 8*(m/4) + 4*(t%2) + m%4
//    so that tiles 2s and 2s+1 together give each lane the 8 consecutive key
//    dims 32s + 8*(l/16) + 0..7 that its Q fragment holds;
//  * score tiles: P^T = K Q^T over 32 keys as two 16-row tiles whose row m
//    is key 8*(m/4) + 4u + m%4 (u = tile), so each lane ends up with the 8
//    consecutive keys 8*(l/16) + 0..7 of one query row, i.e. directly the A
//    operand of P V.
// LDS rows are D + 16 elements long (a stride of 8 mod 32 dwords), which
// spreads both the row reads and the transposing reads over all banks.
// ============================================================================
template <int D>
struct PrefillCfg {
  static constexpr int NW = 4;
  static constexpr int DVW = D / NW;   // value columns per wave
  static constexpr int NDV = DVW / 16; // 16-wide value tiles per wave
  static constexpr int NDK = D / 16;   // 16-row key-dim tiles of the state
  static constexpr int KS = D / 32;    // 32-wide k steps over the head dim
  static constexpr int RS = D + 16;    // LDS row stride (elements)
};

__device__ __forceinline__ int state_row(int t, int m) {
  return 32 * (t >> 1) + 8 * (m >> 2) + 4 * (t & 1) + (m & 3);
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

template <int D>
size_t prefill_bf16_lds_bytes(int C) {
  using Cfg = PrefillCfg<D>;
  const int Cp = (C + 31) & ~31;
  return (size_t)2 * Cp * Cfg::RS * 2;
}

template <int D>
__global__ __launch_bounds__(256, 2) void k_linear_prefill_bf16(
    float* __restrict__ states, int n_slots, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ slots, int H, int C) {
  using Cfg = PrefillCfg<D>;
  constexpr int NDV = Cfg::NDV, NDK = Cfg::NDK, KS = Cfg::KS, RS = Cfg::RS;
  extern __shared__ __align__(16) uint16_t lds_h[];

  const int unit = blockIdx.x;
  const int r = unit / H, h = unit - (unit / H) * H;
  const int tok0 = cu[r], T = cu[r + 1] - tok0;
  const int slot = slots[r];
  if (T <= 0 || slot < 0 || slot >= n_slots) return;

  const int Cp = (C + 31) & ~31;
  uint16_t* Ks = lds_h;
  uint16_t* Vs = Ks + Cp * RS;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
  const int dv0 = w * Cfg::DVW;
  float* S = states + ((int64_t)slot * H + h) * (int64_t)(D * D);
  const int64_t ldx = (int64_t)H * D;
  const uint16_t* qb = q + (int64_t)tok0 * ldx + (int64_t)h * D;
  const uint16_t* kb = k + (int64_t)tok0 * ldx + (int64_t)h * D;
  const uint16_t* vb = v + (int64_t)tok0 * ldx + (int64_t)h * D;
  uint16_t* ob = o + (int64_t)tok0 * ldx + (int64_t)h * D;

  f32x4 Sacc[NDK][NDV];
#pragma unroll
  for (int t = 0; t < NDK; ++t)
#pragma unroll
    for (int n = 0; n < NDV; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Sacc[t][n][i] = S[(int64_t)state_row(t, 4 * lg + i) * D + dv0 + 16 * n + lr];

  for (int c0 = 0; c0 < T; c0 += C) {
    const int n = (T - c0 < C) ? (T - c0) : C;
    __syncthreads();  // the previous chunk's tiles are no longer read
    // ---- stage K and V row-major (rows past n are zero) ----
    {
      constexpr int CG = D / 8;         // 16-byte column groups per row
      constexpr int TGS = 256 / CG;     // 4-token groups per pass
      const int dk8 = tid % CG, tg = tid / CG;
      for (int slab = 0; slab < Cp; slab += 4 * TGS) {
        const int a0 = slab + 4 * tg;
        if (a0 >= Cp) continue;
        u32x4 rk[4], rv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int a = a0 + i;
          if (a < n) {
            const int64_t off = (int64_t)(c0 + a) * ldx + 8 * dk8;
            rk[i] = *reinterpret_cast<const u32x4*>(kb + off);
            rv[i] = *reinterpret_cast<const u32x4*>(vb + off);
          } else {
            rk[i] = u32x4{0u, 0u, 0u, 0u};
            rv[i] = rk[i];
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          *reinterpret_cast<u32x4*>(Ks + (a0 + i) * RS + 8 * dk8) = rk[i];
          *reinterpret_cast<u32x4*>(Vs + (a0 + i) * RS + 8 * dk8) = rv[i];
        }
      }
    }
    __syncthreads();

    // ---- outputs, 16 query rows at a time ----
    // The state registers are not updated before the last row tile, so the
    // bf16 hi/lo B operands of Q S (the state before this chunk) are rebuilt
    // from them per row tile instead of being kept live.
    const int nrt = (n + 15) >> 4;
    // Q fragments come from global memory one row tile ahead of their use
    u32x4 qnext[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qnext[s] = lr < n ? *reinterpret_cast<const u32x4*>(qb + (int64_t)(c0 + lr) * ldx + 32 * s + 8 * lg)
                        : u32x4{0u, 0u, 0u, 0u};
    for (int rt = 0; rt < nrt; ++rt) {
      const int row = 16 * rt + lr;
      u32x4 qf[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) qf[s] = qnext[s];
      if (rt + 1 < nrt) {
        const int nrow = row + 16;
#pragma unroll
        for (int s = 0; s < KS; ++s)
          qnext[s] = nrow < n ? *reinterpret_cast<const u32x4*>(qb + (int64_t)(c0 + nrow) * ldx + 32 * s + 8 * lg)
                              : u32x4{0u, 0u, 0u, 0u};
      }
      f32x4 Oacc[NDV];
#pragma unroll
      for (int nn = 0; nn < NDV; ++nn) {
        Oacc[nn] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          float x[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[i] = Sacc[2 * s][nn][i];
            x[4 + i] = Sacc[2 * s + 1][nn][i];
          }
          u32x4 shi, slo;
          split8(x, shi, slo);
          Oacc[nn] = mfma16x16x32(qf[s], shi, Oacc[nn]);
          Oacc[nn] = mfma16x16x32(qf[s], slo, Oacc[nn]);
        }
      }
      const int nkb = (16 * rt + 15) / 32 + 1;
      for (int kb32 = 0; kb32 < nkb; ++kb32) {
        f32x4 pt[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          pt[u] = f32x4{0.f, 0.f, 0.f, 0.f};
          const int krow = 32 * kb32 + 8 * (lr >> 2) + 4 * u + (lr & 3);
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            const u32x4 kf = *reinterpret_cast<const u32x4*>(Ks + krow * RS + 32 * s + 8 * lg);
            pt[u] = mfma16x16x32(kf, qf[s], pt[u]);
          }
        }
        float pv[8];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = 32 * kb32 + 8 * lg + 4 * u + i;
            pv[4 * u + i] = (key <= row) ? pt[u][i] : 0.f;
          }
        u32x4 phi, plo;
        split8(pv, phi, plo);
#pragma unroll
        for (int nn = 0; nn < NDV; ++nn) {
          const u32x4 vf = tr_operand(Vs, RS, 32 * kb32, dv0 + 16 * nn + 4 * (lr & 3));
          Oacc[nn] = mfma16x16x32(phi, vf, Oacc[nn]);
          Oacc[nn] = mfma16x16x32(plo, vf, Oacc[nn]);
        }
      }
#pragma unroll
      for (int nn = 0; nn < NDV; ++nn)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int orow = 16 * rt + 4 * lg + i;
          if (orow < n)
            ob[(int64_t)(c0 + orow) * ldx + dv0 + 16 * nn + lr] = (uint16_t)f32_to_bf16_bits(Oacc[nn][i]);
        }
    }

    // ---- state update: S += K_c^T V_c ----
    const int nts = (n + 31) >> 5;
    for (int ts = 0; ts < nts; ++ts) {
      u32x4 vf[NDV];
#pragma unroll
      for (int nn = 0; nn < NDV; ++nn) vf[nn] = tr_operand(Vs, RS, 32 * ts, dv0 + 16 * nn + 4 * (lr & 3));
#pragma unroll
      for (int t = 0; t < NDK; ++t) {
        // A operand: K^T rows pi(t, m) = columns of the K tile
        const u32x4 kt = tr_operand(Ks, RS, 32 * ts, 32 * (t >> 1) + 8 * (lr & 3) + 4 * (t & 1));
#pragma unroll
        for (int nn = 0; nn < NDV; ++nn) Sacc[t][nn] = mfma16x16x32(kt, vf[nn], Sacc[t][nn]);
      }
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

template <typename K>
static hipError_t allow_lds(K kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t launch_linear_prefill(float* layer_states, int n_slots, const void* q, const void* k,
                                 const void* v, void* o, const int32_t* cu, const int32_t* slots,
                                 int n_req, int H, int D, int chunk, bool bf16, hipStream_t s) {
  if (n_req <= 0) return hipSuccess;
  dim3 grid((unsigned)(n_req * H)), block(256);
  hipError_t e;
  if (bf16) {
    if (D == 128) {
      const size_t lds = prefill_bf16_lds_bytes<128>(chunk);
      if ((e = allow_lds(k_linear_prefill_bf16<128>, lds)) != hipSuccess) return e;
      hipLaunchKernelGGL(k_linear_prefill_bf16<128>, grid, block, lds, s, layer_states, n_slots,
                         (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                         (uint16_t*)o, cu, slots, H, chunk);
    } else {
      const size_t lds = prefill_bf16_lds_bytes<64>(chunk);
      if ((e = allow_lds(k_linear_prefill_bf16<64>, lds)) != hipSuccess) return e;
      hipLaunchKernelGGL(k_linear_prefill_bf16<64>, grid, block, lds, s, layer_states, n_slots,
                         (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                         (uint16_t*)o, cu, slots, H, chunk);
    }
  } else {
    const size_t lds = (size_t)(D * D + chunk * chunk) * sizeof(float);
    if (D == 128) {
      if ((e = allow_lds(k_linear_prefill_f32<128>, lds)) != hipSuccess) return e;
      hipLaunchKernelGGL(k_linear_prefill_f32<128>, grid, block, lds, s, layer_states, n_slots,
                         (const float*)q, (const float*)k, (const float*)v, (float*)o, cu, slots,
                         H, chunk);
    } else {
      if ((e = allow_lds(k_linear_prefill_f32<64>, lds)) != hipSuccess) return e;
      hipLaunchKernelGGL(k_linear_prefill_f32<64>, grid, block, lds, s, layer_states, n_slots,
                         (const float*)q, (const float*)k, (const float*)v, (float*)o, cu, slots,
                         H, chunk);
    }
  }
  return hipGetLastError();
}

}  // namespace hy
