/*
 * cp_oracle.c -- plain, slow CPU definition of chunked prefill with past.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the graft smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header or table with the
 * HIP library: it includes nothing outside the C standard library and OpenMP.
 *
 * Sources (the four web pages this method is described on):
 *   [SKaiNET]  "functiongemma: chunk prefill-with-past graph
 *               gemma_prefill_with_past" (SKaiNET-transformers PR #417),
 *               sections "Change (additive)" and "Validation".
 *   [TICO]     "Enable prefill-decode modeling" (Samsung/TICO issue #586),
 *               sections "Runtime behavior" and "Mask/cache layout used in
 *               the runtime".
 *   [cactus]   "Pad the chunked-prefill tail for sliding-window models"
 *               (cactus PR #716), sections "Fix" and the review hardening.
 *
 * Precision: attention is accumulated in fp64 with a two-pass softmax.
 * RoPE is evaluated in fp64 on exact fp32 operands (both products are exact
 * in fp64), rounded once to fp32 and then, for bf16 storage, to bf16 by
 * round-to-nearest-even.  Cache updates are byte copies.
 *
 * Storage dtype codes: 0 = fp32, 1 = bf16 (raw 16-bit patterns).
 *
 * A second operator, the gated delta rule of linear-attention layers, follows
 *   [Kazeia]   "Chantier 4 -- GDN chunkwise prefill" (Kazeia-engine docs),
 *               sections "Le kernel actuel" and "P1 -- chunk f32": its
 *               per-token recurrence, evaluated here in fp64 token by token.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_BF16 1

#define ORC_OK 0
#define ORC_EARG (-1)
#define ORC_EWINDOW (-4)
#define ORC_EOVERFLOW (-8)

/* The masked additive value of [SKaiNET] "Change (additive)": 0 attends,
 * -1e30 masks.  It is an fp32 constant added after scaling. */
#define ORC_MASKED (-1e30f)

/* ---------------------------------------------------------------- dtypes */

static float orc_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* fp32 -> bf16, round to nearest, ties to even (NaN kept quiet). */
static uint16_t orc_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

static size_t orc_esize(int dtype) { return dtype == ORC_BF16 ? 2 : 4; }

static double orc_load(const void *base, size_t idx, int dtype) {
  if (dtype == ORC_BF16) return (double)orc_bf16_to_f32(((const uint16_t *)base)[idx]);
  return (double)((const float *)base)[idx];
}

static void orc_store_f32(void *base, size_t idx, float v, int dtype) {
  if (dtype == ORC_BF16)
    ((uint16_t *)base)[idx] = orc_f32_to_bf16(v);
  else
    ((float *)base)[idx] = v;
}

/* ------------------------------------------------------------------ RoPE */

/*
 * Rotary embedding driven by caller-supplied per-position tables
 * ([SKaiNET] "Change (additive)": RoPE from per-position [C, headDim]
 * cos/sin tables; [TICO] "Runtime behavior": (cos_t, sin_t) for the
 * absolute position).  Half-split pairing: element j is paired with
 * j + D/2.
 *
 *   y[j]       = x[j]       * cos[j]       - x[j+D/2] * sin[j]
 *   y[j+D/2]   = x[j+D/2]   * cos[j+D/2]   + x[j]     * sin[j+D/2]
 *
 * x: [B, Hx, C, D] storage dtype; cos/sin: [Bt, C, D] fp32 with Bt in {1, B};
 * y: same shape as x (may alias x).
 */
int orc_rope(const void *x, void *y, const float *cosb, const float *sinb, int B, int Hx,
             int C, int D, int Bt, int dtype) {
  if (!x || !y || !cosb || !sinb || B < 0 || Hx < 0 || C < 0 || D <= 0 || (D & 1)) return ORC_EARG;
  if (Bt != 1 && Bt != B) return ORC_EARG;
  const int h2 = D / 2;
  double *row = (double *)malloc(sizeof(double) * (size_t)D);
  if (!row) return ORC_EARG;
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < Hx; ++h)
      for (int i = 0; i < C; ++i) {
        const size_t xo = (((size_t)b * Hx + h) * C + i) * D;
        const size_t to = ((size_t)(Bt == 1 ? 0 : b) * C + i) * D;
        for (int d = 0; d < D; ++d) row[d] = orc_load(x, xo + d, dtype);
        for (int j = 0; j < h2; ++j) {
          const double lo = row[j], hi = row[j + h2];
          const double ylo = lo * (double)cosb[to + j] - hi * (double)sinb[to + j];
          const double yhi = hi * (double)cosb[to + j + h2] + lo * (double)sinb[to + j + h2];
          orc_store_f32(y, xo + j, (float)ylo, dtype);
          orc_store_f32(y, xo + j + h2, (float)yhi, dtype);
        }
      }
  free(row);
  return ORC_OK;
}

/* ----------------------------------------------------------- cache model */

/*
 * Physical slot of absolute position p.  A global cache stores position p at
 * slot p ([TICO] "Mask/cache layout": past tokens packed into the first
 * past_len slots).  A sliding ring of capacity cap keeps `sink` pinned slots
 * and cycles the remaining cap - sink slots with a write cursor that wraps
 * back to the first non-sink slot.
 */
int orc_slot(int p, int cap, int ring, int sink) {
  if (!ring || p < cap) return p;
  return sink + (p - sink) % (cap - sink);
}

/*
 * Live positions after a sequence has absorbed `seen` positions, in
 * chronological order, by simulating the page's FIFO: [cactus] "Fix" -- the
 * sliding caches compact chronologically on eviction, i.e. each new row
 * pushes out the oldest row that is not a pinned sink row.  A global cache
 * never evicts.  Returns the count written to pos_out (capacity >= cap for a
 * ring, >= seen for a global cache), or ORC_EARG.
 */
int orc_live_positions(int seen, int cap, int ring, int sink, int32_t *pos_out) {
  if (seen < 0 || cap <= 0 || !pos_out) return ORC_EARG;
  if (!ring) {
    for (int p = 0; p < seen; ++p) pos_out[p] = p;
    return seen;
  }
  if (sink < 0 || sink >= cap) return ORC_EARG;
  int n = 0;
  for (int p = 0; p < seen; ++p) {
    pos_out[n++] = p;
    if (n > cap) {
      /* pop the oldest entry that is not a sink position */
      int k = 0;
      while (k < n && pos_out[k] < sink) ++k;
      memmove(pos_out + k, pos_out + k + 1, sizeof(int32_t) * (size_t)(n - k - 1));
      --n;
    }
  }
  return n;
}

/*
 * Append rows [0, n_rows[b]) of the chunk's K/V (rows already rotated, V raw)
 * at positions seen[b], seen[b]+1, ... ([SKaiNET] "Change (additive)": K/V
 * extended by the chunk; [TICO] "Runtime behavior": the runtime writes the
 * delta KV into the external cache).  n_rows == NULL means all C rows.
 *
 * kc, vc: [B, nKV, cap, D] physical images, updated in place on the live
 * region.  seen: [B], updated.  live_out (optional): [B, cap] bytes set to 1
 * where the slot holds a live row after the append.
 * A global cache that would overflow returns ORC_EOVERFLOW and is untouched.
 */
int orc_kv_append(void *kc, void *vc, int32_t *seen, uint8_t *live_out, int B, int nKV, int cap,
                  int D, int dtype, int ring, int sink, const void *kn, const void *vn, int C,
                  const int32_t *n_rows) {
  if (!kc || !vc || !seen || !kn || !vn || B < 0 || nKV <= 0 || cap <= 0 || D <= 0 || C < 0)
    return ORC_EARG;
  if (ring && (sink < 0 || sink >= cap)) return ORC_EARG;
  for (int b = 0; b < B; ++b) {
    const int n = n_rows ? n_rows[b] : C;
    if (n < 0 || n > C || seen[b] < 0) return ORC_EARG;
    if (!ring && seen[b] + n > cap) return ORC_EOVERFLOW;
  }
  const size_t es = orc_esize(dtype);
  const size_t rowb = es * (size_t)D;
  int32_t *before = (int32_t *)malloc(sizeof(int32_t) * (size_t)(cap + C + 1));
  int32_t *after = (int32_t *)malloc(sizeof(int32_t) * (size_t)(cap + C + 1));
  unsigned char *kstage = (unsigned char *)malloc(rowb * (size_t)(cap + C + 1));
  unsigned char *vstage = (unsigned char *)malloc(rowb * (size_t)(cap + C + 1));
  if (!before || !after || !kstage || !vstage) goto fail;
  for (int b = 0; b < B; ++b) {
    const int s0 = seen[b];
    const int n = n_rows ? n_rows[b] : C;
    /* chronological list of live rows before the append */
    int nb;
    if (ring) {
      nb = orc_live_positions(s0, cap, 1, sink, before);
    } else {
      for (int p = 0; p < s0; ++p) before[p] = p;
      nb = s0;
    }
    for (int g = 0; g < nKV; ++g) {
      const size_t cbase = ((size_t)b * nKV + g) * (size_t)cap;
      const size_t nbase = ((size_t)b * nKV + g) * (size_t)C;
      /* FIFO list: positions and their rows */
      int len = 0;
      for (int e = 0; e < nb; ++e) {
        after[len] = before[e];
        const int sl = orc_slot(before[e], cap, ring, sink);
        memcpy(kstage + rowb * len, (const unsigned char *)kc + (cbase + sl) * rowb, rowb);
        memcpy(vstage + rowb * len, (const unsigned char *)vc + (cbase + sl) * rowb, rowb);
        ++len;
      }
      for (int r = 0; r < n; ++r) {
        after[len] = s0 + r;
        memcpy(kstage + rowb * len, (const unsigned char *)kn + (nbase + r) * rowb, rowb);
        memcpy(vstage + rowb * len, (const unsigned char *)vn + (nbase + r) * rowb, rowb);
        ++len;
        if (ring && len > cap) {
          int k = 0;
          while (k < len && after[k] < sink) ++k;
          memmove(after + k, after + k + 1, sizeof(int32_t) * (size_t)(len - k - 1));
          memmove(kstage + rowb * k, kstage + rowb * (k + 1), rowb * (size_t)(len - k - 1));
          memmove(vstage + rowb * k, vstage + rowb * (k + 1), rowb * (size_t)(len - k - 1));
          --len;
        }
      }
      /* write the live rows back at their physical slots */
      for (int e = 0; e < len; ++e) {
        const int sl = orc_slot(after[e], cap, ring, sink);
        memcpy((unsigned char *)kc + (cbase + sl) * rowb, kstage + rowb * e, rowb);
        memcpy((unsigned char *)vc + (cbase + sl) * rowb, vstage + rowb * e, rowb);
      }
      if (live_out && g == 0) {
        memset(live_out + (size_t)b * cap, 0, (size_t)cap);
        for (int e = 0; e < len; ++e) live_out[(size_t)b * cap + orc_slot(after[e], cap, ring, sink)] = 1;
      }
    }
    seen[b] = s0 + n;
  }
  free(before);
  free(after);
  free(kstage);
  free(vstage);
  return ORC_OK;
fail:
  free(before);
  free(after);
  free(kstage);
  free(vstage);
  return ORC_EARG;
}

/*
 * Rows that a padded append of C rows (n_valid real + C - n_valid pad)
 * evicts but an exact append of the n_valid real rows keeps ([cactus] "Fix":
 * a padded append over-evicts up to pad_count of the oldest window rows;
 * snapshot saves them, rollback reinserts them).  Derived here by running
 * both FIFOs and diffing, not from a closed form.
 *
 * Guard ([cactus] review hardening): a ring with window <= chunk + sink is
 * rejected with ORC_EWINDOW.  A global cache never over-evicts (count 0).
 * pos_out needs room for C entries.  Returns the count.
 */
int orc_padded_overevicted(int seen, int n_valid, int C, int cap, int ring, int sink,
                           int32_t *pos_out) {
  if (seen < 0 || C < 0 || n_valid < 0 || n_valid > C || cap <= 0 || !pos_out) return ORC_EARG;
  if (!ring) return 0;
  if (sink < 0 || sink >= cap) return ORC_EARG;
  if (cap <= C + sink) return ORC_EWINDOW;
  int32_t *le = (int32_t *)malloc(sizeof(int32_t) * (size_t)(cap + 1));
  int32_t *lp = (int32_t *)malloc(sizeof(int32_t) * (size_t)(cap + 1));
  if (!le || !lp) {
    free(le);
    free(lp);
    return ORC_EARG;
  }
  const int ne = orc_live_positions(seen + n_valid, cap, 1, sink, le);
  const int np = orc_live_positions(seen + C, cap, 1, sink, lp);
  int cnt = 0;
  for (int a = 0; a < ne; ++a) {
    int found = 0;
    for (int c = 0; c < np; ++c)
      if (lp[c] == le[a]) {
        found = 1;
        break;
      }
    if (!found) pos_out[cnt++] = le[a];
  }
  free(le);
  free(lp);
  return cnt;
}

/* ------------------------------------------------------------- the mask */

/*
 * In-kernel attend rule.  A key at absolute position kp is attended by the
 * query at absolute position qp when it is causal (kp <= qp), is a real row
 * (pad rows of the chunk are never attended: [SKaiNET] "Change (additive)",
 * the mask carries the zero padding), and lies inside the sliding window of
 * W positions counted with the query itself (qp - kp < W), or is a pinned
 * sink row.  W == 0 means no window.
 */
static int orc_attend(long qp, long kp, int key_is_real, int window, int sink) {
  if (!key_is_real || kp > qp) return 0;
  if (window == 0 || qp - kp < window || kp < sink) return 1;
  return 0;
}

/*
 * Explicit additive mask [B, H, C, ld] (fp32; 0 attends, -1e30 masks), laid
 * out as in [SKaiNET] "Change (additive)": one mask row per head and chunk
 * row, columns = the live past rows in chronological order followed by the
 * C chunk rows; columns past L_b + C are masked.  Pad query rows follow the
 * same rule (their outputs are not used).
 */
int orc_build_mask(float *mask, const int32_t *seen, const int32_t *n_valid, int B, int H, int C,
                   long ld, int cap, int ring, int sink, int window) {
  if (!mask || !seen || B < 0 || H <= 0 || C < 0 || ld < 0 || cap <= 0) return ORC_EARG;
  int32_t *pos = (int32_t *)malloc(sizeof(int32_t) * (size_t)(cap + 1));
  if (!pos) return ORC_EARG;
  for (int b = 0; b < B; ++b) {
    const int nv = n_valid ? n_valid[b] : C;
    if (seen[b] < 0 || (!ring && seen[b] > cap)) {
      free(pos);
      return ORC_EARG;
    }
    const int L = orc_live_positions(seen[b], cap, ring, sink, pos);
    if (L < 0 || (long)L + C > ld) {
      free(pos);
      return ORC_EARG;
    }
    for (int h = 0; h < H; ++h)
      for (int i = 0; i < C; ++i) {
        float *mrow = mask + (((size_t)b * H + h) * C + i) * (size_t)ld;
        const long qp = (long)seen[b] + i;
        for (long c = 0; c < ld; ++c) {
          int a;
          if (c < L)
            a = orc_attend(qp, pos[c], 1, window, sink);
          else if (c < L + C)
            a = orc_attend(qp, (long)seen[b] + (c - L), (c - L) < nv, window, sink);
          else
            a = 0;
          mrow[c] = a ? 0.0f : ORC_MASKED;
        }
      }
  }
  free(pos);
  return ORC_OK;
}

/* -------------------------------------------------------------- attention */

/*
 * Grouped-query attention of a chunk over past + C keys ([SKaiNET] "Change
 * (additive)": attnWithPastChunk, heads-first [heads, C, headDim], attention
 * over past + C keys with an additive mask per head).  For sequence b, query
 * head h (KV head g = h / (H / nKV)) and real row i < n_valid[b]:
 *
 *   keys  = live past rows of the cache (chronological), then chunk rows 0..C-1
 *   s_k   = scale * <q_i, k> + m_k      (m_k from `mask`, or the attend rule)
 *   out_i = sum_k softmax(s)_k v_k      (fp64, max-subtracted, two passes)
 *
 * The cache is read as it stands before the chunk is appended.  Rows
 * i >= n_valid[b] (pad rows) are written as zeros.  n_valid == NULL means all
 * C rows are real.  mask == NULL selects the attend rule; otherwise mask
 * element (b, h, i, col) is at mask[b*mbs + h*mhs + i*mld + col].
 *
 * q: [B, H, C, D]; kn, vn: [B, nKV, C, D]; kc, vc: [B, nKV, cap, D], all in
 * the storage dtype.  out: [B, H, C, D] fp64.  rows (optional, [C] bytes):
 * compute only chunk rows i with rows[i] != 0 (others are written as zeros),
 * so that single rows of a large workload can be checked one by one.
 */
int orc_attn(const void *q, const void *kn, const void *vn, const void *kc, const void *vc,
             const int32_t *seen, const int32_t *n_valid, const float *mask, long mld, long mhs,
             long mbs, int B, int H, int nKV, int C, int D, int cap, int ring, int sink, int window,
             float scale, int dtype, const uint8_t *rows, double *out) {
  if (!q || !kn || !vn || !kc || !vc || !seen || !out) return ORC_EARG;
  if (B < 0 || H <= 0 || nKV <= 0 || H % nKV || C < 0 || D <= 0 || cap <= 0) return ORC_EARG;
  const int G = H / nKV;
  /* live past positions per sequence */
  int32_t *pos = (int32_t *)malloc(sizeof(int32_t) * (size_t)B * (size_t)(cap + 1));
  int *L = (int *)malloc(sizeof(int) * (size_t)(B > 0 ? B : 1));
  if (!pos || !L) {
    free(pos);
    free(L);
    return ORC_EARG;
  }
  for (int b = 0; b < B; ++b) {
    if (seen[b] < 0 || (!ring && seen[b] > cap)) {
      free(pos);
      free(L);
      return ORC_EARG;
    }
    L[b] = orc_live_positions(seen[b], cap, ring, sink, pos + (size_t)b * (cap + 1));
    if (L[b] < 0) {
      free(pos);
      free(L);
      return ORC_EARG;
    }
    if (mask && (long)L[b] + C > mld) {
      free(pos);
      free(L);
      return ORC_EARG;
    }
  }
  int rc = ORC_OK;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      const int g = h / G;
      const int nv = n_valid ? n_valid[b] : C;
      const int Lb = L[b];
      const int32_t *pb = pos + (size_t)b * (cap + 1);
      const int nk = Lb + C;
      double *s = (double *)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
      double *qv = (double *)malloc(sizeof(double) * (size_t)D);
      double *acc = (double *)malloc(sizeof(double) * (size_t)D);
      if (!s || !qv || !acc) {
        rc = ORC_EARG;
        free(s);
        free(qv);
        free(acc);
        continue;
      }
      const size_t cbase = ((size_t)b * nKV + g) * (size_t)cap;
      const size_t nbase = ((size_t)b * nKV + g) * (size_t)C;
      for (int i = 0; i < C; ++i) {
        double *o = out + (((size_t)b * H + h) * C + i) * (size_t)D;
        if (i >= nv || (rows && !rows[i])) {
          for (int d = 0; d < D; ++d) o[d] = 0.0;
          continue;
        }
        const size_t qo = (((size_t)b * H + h) * C + i) * (size_t)D;
        for (int d = 0; d < D; ++d) qv[d] = orc_load(q, qo + d, dtype);
        const long qp = (long)seen[b] + i;
        /* pass 1: scores and their maximum */
        double m = -INFINITY;
        for (int c = 0; c < nk; ++c) {
          size_t ko;
          const void *ksrc;
          long kp;
          int real;
          if (c < Lb) {
            kp = pb[c];
            ko = (cbase + (size_t)orc_slot(pb[c], cap, ring, sink)) * (size_t)D;
            ksrc = kc;
            real = 1;
          } else {
            const int j = c - Lb;
            kp = (long)seen[b] + j;
            ko = (nbase + (size_t)j) * (size_t)D;
            ksrc = kn;
            real = j < nv;
          }
          double dot = 0.0;
          for (int d = 0; d < D; ++d) dot += qv[d] * orc_load(ksrc, ko + d, dtype);
          double add;
          if (mask)
            add = (double)mask[(size_t)b * mbs + (size_t)h * mhs + (size_t)i * mld + (size_t)c];
          else
            add = orc_attend(qp, kp, real, window, sink) ? 0.0 : (double)ORC_MASKED;
          s[c] = (double)scale * dot + add;
          if (s[c] > m) m = s[c];
        }
        /* pass 2: normaliser and weighted sum of values */
        double l = 0.0;
        for (int d = 0; d < D; ++d) acc[d] = 0.0;
        for (int c = 0; c < nk; ++c) {
          const double p = exp(s[c] - m);
          if (p == 0.0) continue;
          l += p;
          size_t vo;
          const void *vsrc;
          if (c < Lb) {
            vo = (cbase + (size_t)orc_slot(pb[c], cap, ring, sink)) * (size_t)D;
            vsrc = vc;
          } else {
            vo = (nbase + (size_t)(c - Lb)) * (size_t)D;
            vsrc = vn;
          }
          for (int d = 0; d < D; ++d) acc[d] += p * orc_load(vsrc, vo + d, dtype);
        }
        for (int d = 0; d < D; ++d) o[d] = acc[d] / l;
      }
      free(s);
      free(qv);
      free(acc);
    }
  free(pos);
  free(L);
  return rc;
}

/* -------------------------------------------------------------- selection */

/*
 * Row selection ([SKaiNET] "Change (additive)": LM head on the one-hot
 * selected position; "Validation": select on row 51, the last real row of a
 * 52-token chunk).  y[b, h, :] = x[b, h, idx[b] + off, :], zeros when the
 * row is outside [0, C).
 */
int orc_select_row(const double *x, double *y, const int32_t *idx, int off, int B, int H, int C,
                   int D) {
  if (!x || !y || !idx || B < 0 || H <= 0 || C < 0 || D <= 0) return ORC_EARG;
  for (int b = 0; b < B; ++b) {
    const long r = (long)idx[b] + off;
    for (int h = 0; h < H; ++h)
      for (int d = 0; d < D; ++d)
        y[((size_t)b * H + h) * D + d] =
            (r >= 0 && r < C) ? x[(((size_t)b * H + h) * C + (size_t)r) * D + d] : 0.0;
  }
  return ORC_OK;
}

/* Number of OpenMP threads the oracle runs with (for the CPU baseline). */
int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------ gated delta rule */

/*
 * [Kazeia] "Le kernel actuel" / "P1 -- chunk f32": per (sequence, head) a state S of
 * dk x dv; for every token t, in order:
 *   S <- g_t S                      (gate decay, g_t = exp(alpha_t))
 *   sum = S^T k_t                   (the state's prediction of v_t)
 *   delta = (v_t - sum) * beta_t
 *   S <- S + k_t delta^T            (rank-1 update)
 *   out_t = S^T q_t
 * q, k [B,H,P,dk], v [B,H,P,dv], beta and alpha [B,H,P] (fp32 inputs); s0 [B,H,dk,dv]
 * fp32 initial state (NULL: zero); out [B,H,P,dv] and s_out [B,H,dk,dv] fp64.  The
 * arithmetic is fp64 throughout, serial over the tokens, parallel over (b, h).
 */
int orc_gdn(const float *q, const float *k, const float *v, const float *beta,
            const float *alpha, const float *s0, double *out, double *s_out, int B, int H,
            int P, int dk, int dv) {
  if (B < 0 || H < 0 || P < 0 || dk < 1 || dv < 1) return ORC_EARG;
  if ((long)B * H * P > 0 && (!q || !k || !v || !beta || !alpha || !out)) return ORC_EARG;
  if (!s_out) return ORC_EARG;
  const long nbh = (long)B * H;
#pragma omp parallel for schedule(dynamic)
  for (long bh = 0; bh < nbh; ++bh) {
    double *S = s_out + bh * dk * dv;
    for (long e = 0; e < (long)dk * dv; ++e) S[e] = s0 ? (double)s0[bh * dk * dv + e] : 0.0;
    double *sum = (double *)malloc(sizeof(double) * dv);
    for (int t = 0; t < P; ++t) {
      const long row = bh * P + t;
      const float *kt = k + row * dk, *qt = q + row * dk, *vt = v + row * dv;
      const double g = exp((double)alpha[row]);
      const double bt = (double)beta[row];
      for (long e = 0; e < (long)dk * dv; ++e) S[e] *= g;
      for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += S[(long)i * dv + j] * (double)kt[i];
        sum[j] = acc;
      }
      for (int j = 0; j < dv; ++j) {
        const double delta = ((double)vt[j] - sum[j]) * bt;
        for (int i = 0; i < dk; ++i) S[(long)i * dv + j] += (double)kt[i] * delta;
      }
      double *ot = out + row * dv;
      for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += S[(long)i * dv + j] * (double)qt[i];
        ot[j] = acc;
      }
    }
    free(sum);
  }
  return ORC_OK;
}
