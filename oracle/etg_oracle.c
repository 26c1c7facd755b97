/*
 * CPU oracle for the static embedding / tied lm_head path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  The product path never calls it.
 * It shares no source with the HIP library: its own decoders, its own
 * arithmetic, plain scalar loops, float64 accumulation.
 *
 * What it computes (readings of the pages are listed with each function):
 *
 *   row addressing  HELIX Columnar Embedding proposal, section 3 "Wire format"
 *                   and "Index": row i occupies bytes [i*row_bytes, (i+1)*row_bytes)
 *                   and row_bytes = hidden * itemsize.
 *   gather          ADR-0008 "POST /v1/embed": one f32 row of hidden values per
 *                   token id, looked up by offset; the embeddinggemma.c port
 *                   specification, "Forward graph": x = token_embd[ids] * sqrt(768),
 *                   with the Q8_0 token_embd used by row-gather + dequant only
 *                   ("Tensor inventory").
 *   logits          ADR-0008 "POST /v1/logits": residual @ lm_head.T over every
 *                   vocabulary row, the lm_head tied to the embeddings (ADR-0008
 *                   "Open Questions", item 1; HELIX proposal section 5(a)).
 *   top-k           ADR-0008 "POST /v1/logits": the response lists the top_k
 *                   tokens in descending order.
 *   probabilities   ADR-0008 "POST /v1/logits": each listed token with its
 *                   probability at the request's temperature (softmax of L / T
 *                   over the whole vocabulary).
 *   wire codecs     ADR-0009 "Wire Layout": f16 and per-position symmetric i8
 *                   encodings of residual rows.
 *
 * Every function here has a pin in tests/test_oracle.py against values fixed
 * by the pages or by mathematics; none is "parity unpinned".
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -shared -fPIC (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Storage dtype codes of the oracle's interface.  f16: the embed slice's
 * embeddings.bin stores vocab x hidden binary16 values, decoded per lookup
 * (ADR-0008 "Vindex Slice: embed" and "Memory footprint"). */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_Q8_0 = 2, ORC_F16 = 3 };

/* Q8_0 block: a little-endian binary16 scale, then 32 signed 8-bit values
 * (reading of the "blocks of 32 int8 with one f16 scale" layout; the pages
 * defer the byte layout to an extraction report that is not available). */
#define ORC_Q8_VALUES 32
#define ORC_Q8_BYTES 34

void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Bytes of one stored row: hidden * itemsize for f32 (4), bf16 and f16 (2); for Q8_0,
 * 34 bytes per 32 values.  -1 when the dtype is unknown or hidden does not fit. */
int64_t orc_row_bytes(int dtype, int64_t hidden) {
  if (hidden <= 0) return -1;
  switch (dtype) {
    case ORC_F32: return 4 * hidden;
    case ORC_BF16: return 2 * hidden;
    case ORC_F16: return 2 * hidden;
    case ORC_Q8_0:
      if (hidden % ORC_Q8_VALUES) return -1;
      return (hidden / ORC_Q8_VALUES) * ORC_Q8_BYTES;
    default: return -1;
  }
}

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double orc_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1F;
  int f = h & 0x3FF;
  double mag;
  if (e == 0) {
    mag = ldexp((double)f, -24);                 /* subnormal: f * 2^-14 * 2^-10 */
  } else if (e == 31) {
    mag = f ? NAN : INFINITY;
  } else {
    mag = ldexp((double)(1024 + f), e - 25);     /* (1 + f/2^10) * 2^(e-15) */
  }
  return sign ? -mag : mag;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double orc_bf16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 7) & 0xFF;
  int f = h & 0x7F;
  double mag;
  if (e == 0) {
    mag = ldexp((double)f, -133);                /* subnormal: f * 2^-126 * 2^-7 */
  } else if (e == 255) {
    mag = f ? NAN : INFINITY;
  } else {
    mag = ldexp((double)(128 + f), e - 134);     /* (1 + f/2^7) * 2^(e-127) */
  }
  return sign ? -mag : mag;
}

static uint16_t rd_u16le(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* Decode one stored row into its exact values (every value fits a double exactly). */
void orc_dequant_row(const uint8_t* row, int dtype, int64_t hidden, double* out) {
  int64_t c;
  switch (dtype) {
    case ORC_F32:
      for (c = 0; c < hidden; c++) {
        float v;
        memcpy(&v, row + 4 * c, 4);
        out[c] = (double)v;
      }
      break;
    case ORC_BF16:
      for (c = 0; c < hidden; c++) out[c] = orc_bf16_to_f64(rd_u16le(row + 2 * c));
      break;
    case ORC_F16:
      for (c = 0; c < hidden; c++) out[c] = orc_f16_to_f64(rd_u16le(row + 2 * c));
      break;
    case ORC_Q8_0:
      for (c = 0; c < hidden; c++) {
        const uint8_t* blk = row + (c / ORC_Q8_VALUES) * ORC_Q8_BYTES;
        double s = orc_f16_to_f64(rd_u16le(blk));
        int8_t q = (int8_t)blk[2 + c % ORC_Q8_VALUES];
        out[c] = (double)q * s;
      }
      break;
    default:
      for (c = 0; c < hidden; c++) out[c] = NAN;
  }
}

/* The f32 nearest to sqrt(hidden): the sqrt of a double is correctly rounded and
 * 53 >= 2*24 + 2, so rounding that result to f32 gives the f32 nearest the exact root. */
float orc_sqrt_d(int64_t hidden) { return (float)sqrt((double)hidden); }

/*
 * Gather: out[n][c] = deq(E[ids[n]])[c], or its product with `scale` rounded
 * once to the nearest f32 when use_scale != 0.  The dequantized value is exact
 * in f32 (f32 copy; bf16 widening; int8 * f16 has at most 19 significant bits),
 * and the double product of two f32 values is exact, so one rounding to f32 is
 * the correctly rounded f32 product.  An id that is not in [0, V) as an
 * unsigned 32-bit value gives an all-zero row and is counted.  Returns the
 * number of such ids.
 */
int64_t orc_embed_gather(const uint8_t* table, int dtype, int64_t V, int64_t hidden,
                         const int32_t* ids, int64_t n, float scale, int use_scale, float* out) {
  int64_t rb = orc_row_bytes(dtype, hidden);
  int64_t bad = 0;
  int64_t i;
  if (rb < 0) return -1;
#pragma omp parallel for reduction(+ : bad) schedule(static)
  for (i = 0; i < n; i++) {
    uint32_t id = (uint32_t)ids[i];
    float* o = out + i * hidden;
    int64_t c;
    if ((uint64_t)id >= (uint64_t)V) {
      for (c = 0; c < hidden; c++) o[c] = 0.0f;
      bad += 1;
      continue;
    }
    double* x = (double*)malloc(sizeof(double) * (size_t)hidden);
    orc_dequant_row(table + (uint64_t)id * (uint64_t)rb, dtype, hidden, x);
    for (c = 0; c < hidden; c++) {
      float v = (float)x[c];
      if (use_scale) v = (float)((double)v * (double)scale);
      o[c] = v;
    }
    free(x);
  }
  return bad;
}

/*
 * Logits: L[b][v] = sum_i R[b][i] * deq(E[v])[i], summed in double; every
 * product is exact in double.  A[b][v] = sum_i |R[b][i] * deq(E[v])[i]| is
 * the scale the tolerance is measured against.  No embedding scale, bias,
 * norm or temperature enters here.  L and A are [B][V] row-major; A may be NULL.
 */
void orc_logits(const uint8_t* table, int dtype, int64_t V, int64_t hidden, const float* R,
                int64_t B, double* L, double* A) {
  int64_t rb = orc_row_bytes(dtype, hidden);
  int64_t v;
  if (rb < 0) return;
#pragma omp parallel for schedule(static)
  for (v = 0; v < V; v++) {
    double* x = (double*)malloc(sizeof(double) * (size_t)hidden);
    int64_t b, i;
    orc_dequant_row(table + (uint64_t)v * (uint64_t)rb, dtype, hidden, x);
    for (b = 0; b < B; b++) {
      const float* r = R + b * hidden;
      double s = 0.0, sa = 0.0;
      for (i = 0; i < hidden; i++) {
        double p = (double)r[i] * x[i];
        s += p;
        sa += fabs(p);
      }
      L[b * V + v] = s;
      if (A) A[b * V + v] = sa;
    }
    free(x);
  }
}

/* Order for top-k: larger logit first; equal logits, smaller id first.
 * (-0.0 and +0.0 compare equal, so they tie and fall back to the id.) */
typedef struct {
  double s;
  int32_t id;
} orc_cand;

static int orc_cmp(const void* pa, const void* pb) {
  const orc_cand* a = (const orc_cand*)pa;
  const orc_cand* b = (const orc_cand*)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->id < b->id) ? -1 : (a->id > b->id) ? 1 : 0;
}

/* Top-k of each row of L [B][V]: sort all V (logit, id) pairs by the order above
 * and keep the first k.  scores = the logit rounded to f32. */
void orc_topk(const double* L, int64_t B, int64_t V, int32_t k, int32_t* ids, float* scores) {
  int64_t b;
#pragma omp parallel for schedule(dynamic, 1)
  for (b = 0; b < B; b++) {
    orc_cand* c = (orc_cand*)malloc(sizeof(orc_cand) * (size_t)V);
    int64_t v;
    int32_t j;
    for (v = 0; v < V; v++) {
      c[v].s = L[b * V + v];
      c[v].id = (int32_t)v;
    }
    qsort(c, (size_t)V, sizeof(orc_cand), orc_cmp);
    for (j = 0; j < k; j++) {
      ids[b * k + j] = c[j].id;
      scores[b * k + j] = (float)c[j].s;
    }
    free(c);
  }
}

/* Logits of selected (b, id) pairs only, for spot checks at full size:
 * out_L[j] = L[b_j][id_j], out_A[j] = A[b_j][id_j]. */
void orc_logits_at(const uint8_t* table, int dtype, int64_t V, int64_t hidden, const float* R,
                   const int64_t* bs, const int32_t* vids, int64_t npairs, double* out_L, double* out_A) {
  int64_t rb = orc_row_bytes(dtype, hidden);
  int64_t j;
  if (rb < 0) return;
#pragma omp parallel for schedule(static)
  for (j = 0; j < npairs; j++) {
    double* x = (double*)malloc(sizeof(double) * (size_t)hidden);
    const float* r = R + bs[j] * hidden;
    double s = 0.0, sa = 0.0;
    int64_t i;
    uint32_t v = (uint32_t)vids[j];
    if ((uint64_t)v >= (uint64_t)V) {
      out_L[j] = NAN;
      out_A[j] = NAN;
      free(x);
      continue;
    }
    orc_dequant_row(table + (uint64_t)v * (uint64_t)rb, dtype, hidden, x);
    for (i = 0; i < hidden; i++) {
      double p = (double)r[i] * x[i];
      s += p;
      sa += fabs(p);
    }
    out_L[j] = s;
    out_A[j] = sa;
    free(x);
  }
}

/*
 * Probabilities at a temperature (ADR-0008 "POST /v1/logits": each listed token
 * carries its probability at the request's temperature).  Reading: the softmax
 * of L / T over the whole vocabulary, so the listed probabilities are those of
 * the full distribution (they need not sum to 1 over the top k).
 *
 *   lse[b] = log(sum_v exp(L[b][v] / T))
 *          = M / T + log(sum_v exp((L[b][v] - M) / T)),  M = max_v L[b][v]
 *
 * (the shift by M is an identity that keeps every exp argument <= 0).  The sum
 * runs in double in vocabulary order.  T > 0.
 */
void orc_log_partition(const double* L, int64_t B, int64_t V, double T, double* lse) {
  int64_t b;
#pragma omp parallel for schedule(static)
  for (b = 0; b < B; b++) {
    const double* x = L + b * V;
    double m = x[0], s = 0.0;
    int64_t v;
    for (v = 1; v < V; v++)
      if (x[v] > m) m = x[v];
    for (v = 0; v < V; v++) s += exp((x[v] - m) / T);
    lse[b] = m / T + log(s);
  }
}

/* prob[b][j] = exp(L[b][ids[b][j]] / T - lse[b]) for k ids per row (NAN for an id
 * outside [0, V)). */
void orc_probs_at(const double* L, const double* lse, int64_t B, int64_t V, double T, const int32_t* ids,
                  int32_t k, double* prob) {
  int64_t b;
  int32_t j;
  for (b = 0; b < B; b++)
    for (j = 0; j < k; j++) {
      const uint32_t v = (uint32_t)ids[b * k + j];
      prob[b * k + j] = (uint64_t)v < (uint64_t)V ? exp(L[b * V + v] / T - lse[b]) : NAN;
    }
}

/*
 * Residual wire codecs (ADR-0009 "Wire Layout"): the embed output and the
 * logits input may travel as
 *   wire 0  f32: hidden little-endian binary32 values per row (4 hidden bytes);
 *   wire 1  f16: hidden little-endian binary16 values per row (2 hidden bytes);
 *   wire 2  i8 symmetric, per position: [scale f32][zero_point f32 = 0]
 *           [hidden int8] (hidden + 8 bytes), scale = max|x| / 127 and
 *           x^ = q * scale.
 * Readings: f16 rounds to nearest even and clamps to +-65504 (the page's
 * clamp-to-max overflow); the i8 code is q = round-half-even(x / scale) taken
 * in f32, as are max|x| and scale = max|x| / 127.0f (the codes are integers
 * decided by floating point, so both sides decide in f32), clamped to
 * [-127, 127]; a row with scale 0 encodes as all zeros.
 */
enum { ORC_WIRE_F32 = 0, ORC_WIRE_F16 = 1, ORC_WIRE_I8 = 2 };

int64_t orc_wire_row_bytes(int wire, int64_t hidden) {
  switch (wire) {
    case ORC_WIRE_F32: return 4 * hidden;
    case ORC_WIRE_F16: return 2 * hidden;
    case ORC_WIRE_I8: return hidden + 8;
    default: return -1;
  }
}

/* Round-half-even of a non-negative double holding an exact small value. */
static double orc_rne(double m) {
  double f = floor(m), d = m - f;
  if (d > 0.5) return f + 1.0;
  if (d < 0.5) return f;
  return fmod(f, 2.0) == 0.0 ? f : f + 1.0;
}

/* Nearest binary16 (ties to even) of a finite float, clamped to +-65504. */
uint16_t orc_f32_to_f16_sat(float x) {
  const uint16_t sign = signbit(x) ? 0x8000 : 0;
  const double a = fabs((double)x);
  int ex;
  double q;
  if (a >= 65504.0) return sign | 0x7BFF;
  if (a < ldexp(1.0, -14)) {
    /* subnormal range: multiples of 2^-24; q = 1024 is the smallest normal */
    q = orc_rne(ldexp(a, 24));
    return sign | (uint16_t)q;
  }
  frexp(a, &ex);                           /* a = m 2^ex, m in [0.5, 1) */
  ex -= 1;                                 /* a in [2^ex, 2^(ex+1)), ex >= -14 */
  q = orc_rne(ldexp(a, 10 - ex));          /* in [1024, 2048] */
  if (q == 2048.0) {
    q = 1024.0;
    ex += 1;
  }
  if (ex + 15 >= 31) return sign | 0x7BFF; /* cannot happen below 65504 */
  return sign | (uint16_t)(((ex + 15) << 10) | ((int)q - 1024));
}

/* Encode n rows of hidden f32 values into wire rows (orc_wire_row_bytes each). */
void orc_wire_encode(const float* x, int64_t n, int64_t hidden, int wire, uint8_t* out) {
  const int64_t rb = orc_wire_row_bytes(wire, hidden);
  int64_t r, c;
  for (r = 0; r < n; r++) {
    const float* xr = x + r * hidden;
    uint8_t* o = out + r * rb;
    if (wire == ORC_WIRE_F32) {
      memcpy(o, xr, (size_t)(4 * hidden));
    } else if (wire == ORC_WIRE_F16) {
      for (c = 0; c < hidden; c++) {
        const uint16_t h = orc_f32_to_f16_sat(xr[c]);
        o[2 * c] = (uint8_t)(h & 0xFF);
        o[2 * c + 1] = (uint8_t)(h >> 8);
      }
    } else {
      float m = 0.0f, scale, zero = 0.0f;
      for (c = 0; c < hidden; c++)
        if (fabsf(xr[c]) > m) m = fabsf(xr[c]);
      scale = m / 127.0f;
      memcpy(o, &scale, 4);
      memcpy(o + 4, &zero, 4);
      for (c = 0; c < hidden; c++) {
        float q = 0.0f;
        if (scale != 0.0f) {
          q = rintf(xr[c] / scale);
          if (q > 127.0f) q = 127.0f;
          if (q < -127.0f) q = -127.0f;
        }
        o[8 + c] = (uint8_t)(int8_t)q;
      }
    }
  }
}

/* Decode n wire rows into f32 values: f16 widened exactly, i8 as q * scale (one
 * f32 rounding). */
void orc_wire_decode(const uint8_t* in, int64_t n, int64_t hidden, int wire, float* out) {
  const int64_t rb = orc_wire_row_bytes(wire, hidden);
  int64_t r, c;
  for (r = 0; r < n; r++) {
    const uint8_t* row = in + r * rb;
    float* o = out + r * hidden;
    if (wire == ORC_WIRE_F32) {
      memcpy(o, row, (size_t)(4 * hidden));
    } else if (wire == ORC_WIRE_F16) {
      for (c = 0; c < hidden; c++) o[c] = (float)orc_f16_to_f64(rd_u16le(row + 2 * c));
    } else {
      float scale;
      memcpy(&scale, row, 4);
      for (c = 0; c < hidden; c++) o[c] = (float)(int8_t)row[8 + c] * scale;
    }
  }
}

/* Element-wise decoders over arrays (for the decoder pins). */
void orc_f16_array(const uint16_t* h, int64_t n, double* out) {
  int64_t i;
  for (i = 0; i < n; i++) out[i] = orc_f16_to_f64(h[i]);
}

void orc_bf16_array(const uint16_t* h, int64_t n, double* out) {
  int64_t i;
  for (i = 0; i < n; i++) out[i] = orc_bf16_to_f64(h[i]);
}
