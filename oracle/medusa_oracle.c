/*
 * medusa_oracle.c -- plain, slow, fp64 CPU reference for one Medusa verification step.
 *
 * TEST INFRASTRUCTURE ONLY.  The parity tests, the smoke check and the benchmark's CPU
 * baseline are the only callers.  The HIP library never links, loads or calls this code, and
 * this file includes nothing of it.
 *
 * Every input element is read in its stored type (fp32, or bf16 held as a uint16 bit pattern)
 * and widened to double; all arithmetic is double with sequential sums in index order.  OpenMP
 * (when enabled) only splits independent output rows or (batch, head, node) units across
 * threads; it never reorders a sum.
 *
 * Sources (page titles as printed in the page headers):
 *  - heads: Ultralytics glossary "Medusa Heads", section on how the heads predict the next
 *    tokens: each head is one fully connected layer with SiLU and a residual connection,
 *    followed by a vocab projection; its code sample builds Linear(hidden, hidden) with a bias
 *    and Linear(hidden, vocab) without one, and applies out(h + silu(layer(h))).
 *  - tree attention: Wiblog "Medusa multi-head speculative decoding", tree-attention section:
 *    each token attends only to the tokens on its own prefix path; Ultralytics page,
 *    tree-attention section: the mask lets each token see only its ancestors in the tree.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define DT_F32 0
#define DT_BF16 1

static double ld(const void* p, int dt, size_t i) {
  if (dt == DT_F32) return (double)((const float*)p)[i];
  uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/*
 * out[b*out_stride + v] = sum_j W[v][j] * x[b*x_stride + j]   for b < B, v < rows.
 * W is [rows][hd] (torch Linear layout [out,in]); no bias.
 */
void oracle_project(const void* w, int dt, long rows, int hd, const double* x, long x_stride,
                    int B, double* out, long out_stride) {
  long v;
#pragma omp parallel for schedule(static)
  for (v = 0; v < rows; ++v) {
    for (int b = 0; b < B; ++b) {
      double s = 0.0;
      for (int j = 0; j < hd; ++j)
        s += ld(w, dt, (size_t)v * hd + j) * x[(size_t)b * x_stride + j];
      out[(size_t)b * out_stride + v] = s;
    }
  }
}

/*
 * One Medusa head per k, applied to the same last hidden state h[b]:
 *   u      = W1[k] h + b1[k]
 *   r[b,k] = h + SiLU(u),   SiLU(u) = u / (1 + exp(-u))
 *   logits[b,k,:] = W2[k] r[b,k]          (the same projection routine as any LM head)
 * h [B][hd]; w1 [K][hd][hd]; b1 [K][hd]; w2 [K][V][hd]; r [B][K][hd]; logits [B][K][V].
 */
void oracle_heads(const void* h, const void* w1, const void* b1, const void* w2, int dt, int B,
                  int hd, long V, int K, double* r, double* logits) {
  size_t es = dt == DT_F32 ? 4 : 2;
  for (int k = 0; k < K; ++k) {
    for (int b = 0; b < B; ++b) {
      int i;
#pragma omp parallel for schedule(static)
      for (i = 0; i < hd; ++i) {
        double u = 0.0;
        for (int j = 0; j < hd; ++j)
          u += ld(w1, dt, ((size_t)k * hd + i) * hd + j) * ld(h, dt, (size_t)b * hd + j);
        u += ld(b1, dt, (size_t)k * hd + i);
        r[((size_t)b * K + k) * hd + i] = ld(h, dt, (size_t)b * hd + i) + u / (1.0 + exp(-u));
      }
    }
  }
  for (int k = 0; k < K; ++k)
    oracle_project((const char*)w2 + (size_t)k * V * hd * es, dt, V, hd, r + (size_t)k * hd,
                   (long)K * hd, B, logits + (size_t)k * V, (long)K * V);
}

/*
 * Top-k of each row of x [rows][n]: the k largest values, in descending order; equal values go
 * to the lower index.  Plain repeated selection: pick the best not yet taken, k times.
 */
void oracle_topk(const double* x, long rows, long n, int k, int32_t* ids, double* vals) {
  long row;
#pragma omp parallel for schedule(static)
  for (row = 0; row < rows; ++row) {
    const double* xr = x + (size_t)row * n;
    for (int t = 0; t < k; ++t) {
      long best = -1;
      for (long v = 0; v < n; ++v) {
        int taken = 0;
        for (int u = 0; u < t; ++u)
          if (ids[(size_t)row * k + u] == v) taken = 1;
        if (taken) continue;
        if (best < 0 || xr[v] > xr[best]) best = v;
      }
      ids[(size_t)row * k + t] = (int32_t)best;
      if (vals) vals[(size_t)row * k + t] = best >= 0 ? xr[best] : -INFINITY;
    }
  }
}

/* scale * q . k for one query vector and one cache row */
static double score(const void* q, const void* kc, int dt, size_t qoff, size_t krow, int D,
                    double scale) {
  double s = 0.0;
  for (int d = 0; d < D; ++d) s += ld(q, dt, qoff + d) * ld(kc, dt, krow * D + d);
  return s * scale;
}

static int mask_bit(const uint64_t* mask, int W, int i, int t) {
  return (int)((mask[(size_t)i * W + t / 64] >> (t % 64)) & 1ull);
}

/*
 * Tree-masked attention, one output vector per (b, q-head hq, tree node i):
 *   kv head g = hq / (Hq / Hkv)
 *   visible cache rows: every prefix row j < prefix_len[b], and row prefix_len[b] + t for every
 *   tree node t whose bit is set in mask row i (bit t%64 of word t/64);
 *   s_j = scale * q . k_j,  w_j = exp(s_j - max s),  out = sum_j w_j v_j / sum_j w_j.
 * q/out [B][Hq][T][D]; caches [B][Hkv][lcap][D]; mask [T][W] uint64; D <= 256.
 * sel: optional list of nsel (b, hq, i) triples; when NULL every unit is computed.  Units not
 * selected are left untouched in out.
 */
void oracle_tree_attention(const void* q, const void* kc, const void* vc, int dt,
                           const int32_t* prefix_len, int B, int Hq, int Hkv, int T, int D,
                           long lcap, const uint64_t* mask, int W, double scale,
                           const int32_t* sel, long nsel, double* out) {
  long nunits = sel ? nsel : (long)B * Hq * T;
  long u;
#pragma omp parallel for schedule(dynamic, 1)
  for (u = 0; u < nunits; ++u) {
    int b, hq, i;
    if (sel) {
      b = sel[3 * u];
      hq = sel[3 * u + 1];
      i = sel[3 * u + 2];
    } else {
      b = (int)(u / ((long)Hq * T));
      hq = (int)((u / T) % Hq);
      i = (int)(u % T);
    }
    int g = hq / (Hq / Hkv);
    long L = prefix_len[b];
    size_t qoff = (((size_t)b * Hq + hq) * T + i) * D;
    size_t base = ((size_t)b * Hkv + g) * lcap; /* cache row 0 of this (b, g) */

    double smax = -INFINITY;
    for (long j = 0; j < L; ++j) {
      double s = score(q, kc, dt, qoff, base + j, D, scale);
      if (s > smax) smax = s;
    }
    for (int t = 0; t < T; ++t) {
      if (!mask_bit(mask, W, i, t)) continue;
      double s = score(q, kc, dt, qoff, base + L + t, D, scale);
      if (s > smax) smax = s;
    }

    double den = 0.0, acc[256];
    for (int d = 0; d < D; ++d) acc[d] = 0.0;
    for (long j = 0; j < L + T; ++j) {
      if (j >= L && !mask_bit(mask, W, i, (int)(j - L))) continue;
      double w = exp(score(q, kc, dt, qoff, base + j, D, scale) - smax);
      den += w;
      for (int d = 0; d < D; ++d) acc[d] += w * ld(vc, dt, (base + j) * D + d);
    }
    for (int d = 0; d < D; ++d) out[qoff + d] = acc[d] / den;
  }
}
