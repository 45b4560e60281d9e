/*
 * hyattn_ref -- plain, slow, fp64 CPU oracle for the per-layer attention step
 * of a hybrid full/linear-attention model.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the bench's
 * CPU-baseline leg may load this library. The product path never calls it and
 * shares no code, header, table or helper with it.
 *
 * Sources (cited by page title and section; "P2" below is the page
 * "推理框架适配Hybrid Model：KV Cache管理与算子调度实战", "P1" the page
 * "Hybrid Model推理适配：vLLM与SGLang的工程实践指南"):
 *   - P2 §2.1: a linear-attention layer keeps a state matrix (D x D per head);
 *     each new token adds the outer product k (x) v to it and the layer's
 *     output is q times the state. Per-step decode cost is O(D^2).
 *   - P2 §2.1: full-attention KV is cut into fixed 16-token blocks, mapped to
 *     physical memory through a per-request page (block) table.
 *   - P2 §2.3: full layers are softmax attention over Q, K, V and the block
 *     table; linear layers map (Q, K, V, previous state) to (output, new state).
 *   - P2 §2.4: chunked prefill keeps the linear state between chunks; chunk
 *     boundaries must not shift it.
 *
 * Readings of points the pages leave open (each is listed with its reason in
 * the design notes of the repository):
 *   - update then read ("inclusive"): token t's output uses the state that
 *     already contains k_t (x) v_t;
 *   - S[i][j] += k[i] * v[j]  (row = key dim, column = value dim) and
 *     o[j] = sum_i q[i] * S[i][j];
 *   - identity feature map, no normaliser, no extra scale; no decay in the
 *     plain layer (the gated variant below adds a per-token forget factor);
 *   - logical token p of a request lives in physical block table[p / 16] at
 *     offset p % 16; a pool is laid out [n_blocks][H_kv][16][D];
 *   - query head h reads KV head h / (H_q / H_kv).
 *
 * Inputs may be stored as float32, bfloat16 (raw 16-bit patterns) or float64;
 * they are widened exactly to double. All arithmetic is double, in the plain
 * order written below; there is no blocking, fusion or reordering.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define REF_F32 0
#define REF_BF16 1
#define REF_F64 2

static double ld(const void* p, int dt, int64_t i) {
  if (dt == REF_F32) return (double)((const float*)p)[i];
  if (dt == REF_BF16) {
    uint32_t b = (uint32_t)((const uint16_t*)p)[i] << 16;
    float f;
    memcpy(&f, &b, sizeof f);
    return (double)f;
  }
  return ((const double*)p)[i];
}

int ref_abi_version(void) { return 1; }

/* ---------------------------------------------------------------------------
 * Linear attention, token by token -- the definition (P2 §2.1).
 *
 * One (request, head) unit of T tokens. Token t's q/k/v row starts at element
 * `off + t * ldx` of the q/k/v arrays (D contiguous elements). S is the D x D
 * state in row-major double, read as the prior state and overwritten with the
 * final one. Output row t is written at o + t * ldo.
 */
void ref_linear_recurrent(int T, int D, int dt, const void* q, const void* k,
                          const void* v, int64_t off, int64_t ldx, double* S,
                          double* o, int64_t ldo) {
  for (int t = 0; t < T; ++t) {
    const int64_t row = off + (int64_t)t * ldx;
    /* state update: S <- S + k (x) v */
    for (int i = 0; i < D; ++i) {
      const double ki = ld(k, dt, row + i);
      for (int j = 0; j < D; ++j) S[(int64_t)i * D + j] += ki * ld(v, dt, row + j);
    }
    /* output: o = q . S (with the updated state) */
    for (int j = 0; j < D; ++j) {
      double acc = 0.0;
      for (int i = 0; i < D; ++i) acc += ld(q, dt, row + i) * S[(int64_t)i * D + j];
      o[(int64_t)t * ldo + j] = acc;
    }
  }
}

/* ---------------------------------------------------------------------------
 * Linear attention, chunked (P2 §2.4: the state is carried from chunk to
 * chunk). For each chunk of C tokens (the last may be shorter), starting from
 * the state S0 of everything before the chunk:
 *     out_a = q_a . S0 + sum_{b <= a in chunk} (q_a . k_b) v_b
 *     S0   <- S0 + sum_{b in chunk} k_b (x) v_b
 * which equals the token recurrence in exact arithmetic.
 */
void ref_linear_chunked(int T, int C, int D, int dt, const void* q, const void* k,
                        const void* v, int64_t off, int64_t ldx, double* S,
                        double* o, int64_t ldo) {
  if (C < 1) C = 1;
  double* P = (double*)malloc(sizeof(double) * (size_t)C * (size_t)C);
  for (int c0 = 0; c0 < T; c0 += C) {
    const int n = (T - c0 < C) ? (T - c0) : C;
    /* intra-chunk scores, causal with the diagonal included */
    for (int a = 0; a < n; ++a)
      for (int b = 0; b < n; ++b) {
        double s = 0.0;
        if (b <= a) {
          const int64_t ra = off + (int64_t)(c0 + a) * ldx;
          const int64_t rb = off + (int64_t)(c0 + b) * ldx;
          for (int i = 0; i < D; ++i) s += ld(q, dt, ra + i) * ld(k, dt, rb + i);
        }
        P[(int64_t)a * C + b] = s;
      }
    /* outputs: inter-chunk part from S0, intra-chunk part from P */
    for (int a = 0; a < n; ++a) {
      const int64_t ra = off + (int64_t)(c0 + a) * ldx;
      for (int j = 0; j < D; ++j) {
        double acc = 0.0;
        for (int i = 0; i < D; ++i) acc += ld(q, dt, ra + i) * S[(int64_t)i * D + j];
        for (int b = 0; b <= a; ++b)
          acc += P[(int64_t)a * C + b] * ld(v, dt, off + (int64_t)(c0 + b) * ldx + j);
        o[(int64_t)(c0 + a) * ldo + j] = acc;
      }
    }
    /* state update by the whole chunk */
    for (int i = 0; i < D; ++i)
      for (int j = 0; j < D; ++j) {
        double acc = 0.0;
        for (int b = 0; b < n; ++b) {
          const int64_t rb = off + (int64_t)(c0 + b) * ldx;
          acc += ld(k, dt, rb + i) * ld(v, dt, rb + j);
        }
        S[(int64_t)i * D + j] += acc;
      }
  }
  free(P);
}

/* ---------------------------------------------------------------------------
 * Linear attention, closed form over the whole sequence (no softmax, causal
 * mask including the diagonal):
 *     out_t = q_t . S0 + sum_{u <= t} (q_t . k_u) v_u,   S_T = S0 + sum_u k_u (x) v_u
 * S holds S0 on entry and S_T on return.
 */
void ref_linear_closed_form(int T, int D, int dt, const void* q, const void* k,
                            const void* v, int64_t off, int64_t ldx, double* S,
                            double* o, int64_t ldo) {
  for (int t = 0; t < T; ++t) {
    const int64_t rt = off + (int64_t)t * ldx;
    for (int j = 0; j < D; ++j) {
      double acc = 0.0;
      for (int i = 0; i < D; ++i) acc += ld(q, dt, rt + i) * S[(int64_t)i * D + j];
      o[(int64_t)t * ldo + j] = acc;
    }
    for (int u = 0; u <= t; ++u) {
      const int64_t ru = off + (int64_t)u * ldx;
      double s = 0.0;
      for (int i = 0; i < D; ++i) s += ld(q, dt, rt + i) * ld(k, dt, ru + i);
      for (int j = 0; j < D; ++j) o[(int64_t)t * ldo + j] += s * ld(v, dt, ru + j);
    }
  }
  for (int i = 0; i < D; ++i)
    for (int j = 0; j < D; ++j) {
      double acc = 0.0;
      for (int u = 0; u < T; ++u) {
        const int64_t ru = off + (int64_t)u * ldx;
        acc += ld(k, dt, ru + i) * ld(v, dt, ru + j);
      }
      S[(int64_t)i * D + j] += acc;
    }
}

/* ---------------------------------------------------------------------------
 * Decayed (gated) linear attention: the state recurrence with a forget factor,
 * the nearest relative of the linear layer among the state-update variants the
 * pages point to (P2 §1.3: Mamba- and RWKV-style layers; P1 §2.1: a state
 * carried as h_t = f(h_{t-1}, x_t)). Token t brings a log forget factor
 * g_t <= 0 for its head, gamma_t = exp(g_t), and
 *     S_t = gamma_t S_{t-1} + k_t (x) v_t,   out_t = q_t . S_t.
 * g_t = 0 everywhere is the plain linear layer above. g of token t is read at
 * element goff + t * ldg of g (type dt_g).
 */
void ref_linear_gated_recurrent(int T, int D, int dt, const void* q, const void* k,
                                const void* v, int64_t off, int64_t ldx, int dt_g,
                                const void* g, int64_t goff, int64_t ldg, double* S,
                                double* o, int64_t ldo) {
  for (int t = 0; t < T; ++t) {
    const int64_t row = off + (int64_t)t * ldx;
    const double gamma = exp(ld(g, dt_g, goff + (int64_t)t * ldg));
    for (int i = 0; i < D; ++i) {
      const double ki = ld(k, dt, row + i);
      for (int j = 0; j < D; ++j) {
        double* s = &S[(int64_t)i * D + j];
        *s = gamma * *s + ki * ld(v, dt, row + j);
      }
    }
    for (int j = 0; j < D; ++j) {
      double acc = 0.0;
      for (int i = 0; i < D; ++i) acc += ld(q, dt, row + i) * S[(int64_t)i * D + j];
      o[(int64_t)t * ldo + j] = acc;
    }
  }
}

/*
 * The same, chunk by chunk (P2 §2.4). Within a chunk starting from S0, let
 * L_a = g_0 + ... + g_a (positions relative to the chunk). Unrolling the
 * recurrence gives
 *     out_a = exp(L_a) q_a . S0 + sum_{b <= a} exp(L_a - L_b) (q_a . k_b) v_b
 *     S0   <- exp(L_last) S0 + sum_b exp(L_last - L_b) k_b (x) v_b
 * All factors are exp of a sum of g's, so none exceeds 1.
 */
void ref_linear_gated_chunked(int T, int C, int D, int dt, const void* q, const void* k,
                              const void* v, int64_t off, int64_t ldx, int dt_g,
                              const void* g, int64_t goff, int64_t ldg, double* S,
                              double* o, int64_t ldo) {
  if (C < 1) C = 1;
  double* P = (double*)malloc(sizeof(double) * (size_t)C * (size_t)C);
  double* L = (double*)malloc(sizeof(double) * (size_t)C);
  for (int c0 = 0; c0 < T; c0 += C) {
    const int n = (T - c0 < C) ? (T - c0) : C;
    double run = 0.0;
    for (int a = 0; a < n; ++a) {
      run += ld(g, dt_g, goff + (int64_t)(c0 + a) * ldg);
      L[a] = run;
    }
    for (int a = 0; a < n; ++a)
      for (int b = 0; b < n; ++b) {
        double s = 0.0;
        if (b <= a) {
          const int64_t ra = off + (int64_t)(c0 + a) * ldx;
          const int64_t rb = off + (int64_t)(c0 + b) * ldx;
          for (int i = 0; i < D; ++i) s += ld(q, dt, ra + i) * ld(k, dt, rb + i);
          s *= exp(L[a] - L[b]);
        }
        P[(int64_t)a * C + b] = s;
      }
    for (int a = 0; a < n; ++a) {
      const int64_t ra = off + (int64_t)(c0 + a) * ldx;
      const double da = exp(L[a]);
      for (int j = 0; j < D; ++j) {
        double inter = 0.0;
        for (int i = 0; i < D; ++i) inter += ld(q, dt, ra + i) * S[(int64_t)i * D + j];
        double acc = da * inter;
        for (int b = 0; b <= a; ++b)
          acc += P[(int64_t)a * C + b] * ld(v, dt, off + (int64_t)(c0 + b) * ldx + j);
        o[(int64_t)(c0 + a) * ldo + j] = acc;
      }
    }
    const double dn = exp(L[n - 1]);
    for (int i = 0; i < D; ++i)
      for (int j = 0; j < D; ++j) {
        double acc = 0.0;
        for (int b = 0; b < n; ++b) {
          const int64_t rb = off + (int64_t)(c0 + b) * ldx;
          acc += exp(L[n - 1] - L[b]) * ld(k, dt, rb + i) * ld(v, dt, rb + j);
        }
        S[(int64_t)i * D + j] = dn * S[(int64_t)i * D + j] + acc;
      }
  }
  free(L);
  free(P);
}

/* ---------------------------------------------------------------------------
 * Paged KV addressing (P2 §2.1 page table of 16-token blocks).
 * Element offset of logical token p of KV head g in a pool laid out
 * [n_blocks][H_kv][16][D]; -1 if the table has no block for it.
 */
int64_t ref_kv_offset(const int32_t* block_table, int p, int H_kv, int g, int D) {
  const int32_t blk = block_table[p / 16];
  if (blk < 0) return -1;
  return (((int64_t)blk * H_kv + g) * 16 + (p % 16)) * (int64_t)D;
}

/* ---------------------------------------------------------------------------
 * Full attention for one query vector over the first n_keys logical tokens of
 * one request (P2 §2.3: softmax attention over the cached K/V reached through
 * the block table). scores_p = scale * (q . k_p); out = softmax(scores) . V,
 * evaluated with the maximum subtracted before exp. n_keys == 0 gives zeros.
 * q is D elements at q + q_off. Returns 0, or -1 if a needed block is missing.
 */
int ref_paged_attention_query(int D, int dt_q, const void* q, int64_t q_off,
                              int dt_kv, const void* k_pool, const void* v_pool,
                              int H_kv, int g, const int32_t* block_table,
                              int n_keys, double scale, double* out) {
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  if (n_keys <= 0) return 0;
  double* s = (double*)malloc(sizeof(double) * (size_t)n_keys);
  double m = -INFINITY;
  for (int p = 0; p < n_keys; ++p) {
    const int64_t ko = ref_kv_offset(block_table, p, H_kv, g, D);
    if (ko < 0) { free(s); return -1; }
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += ld(q, dt_q, q_off + d) * ld(k_pool, dt_kv, ko + d);
    s[p] = scale * dot;
    if (s[p] > m) m = s[p];
  }
  double den = 0.0;
  for (int p = 0; p < n_keys; ++p) {
    s[p] = exp(s[p] - m);
    den += s[p];
  }
  for (int p = 0; p < n_keys; ++p) {
    const int64_t vo = ref_kv_offset(block_table, p, H_kv, g, D);
    const double w = s[p] / den;
    for (int d = 0; d < D; ++d) out[d] += w * ld(v_pool, dt_kv, vo + d);
  }
  free(s);
  return 0;
}
