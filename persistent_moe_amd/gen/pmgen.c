/* Seeded, element-addressable input generator: a C transcription of the
 * definition in persistent_moe_amd/workloads.py, used to draw large inputs on
 * the host quickly.  It holds none of the decode arithmetic.
 *
 * fmix32 is the 32-bit finaliser of MurmurHash3 (Austin Appleby, public
 * domain).  The float steps use only +, -, *, /, sqrt and frexp, all exact or
 * correctly rounded in IEEE double, evaluated in the same order as the
 * Python definition; the file is built with -ffp-contract=off so that no
 * multiply-add is fused.  The outputs are therefore bit-identical to the
 * numpy and torch versions of the definition.
 */
#include <math.h>
#include <stdint.h>

static inline uint32_t fmix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85EBCA6Bu;
  h ^= h >> 13;
  h *= 0xC2B2AE35u;
  h ^= h >> 16;
  return h;
}

static const double LN2 = 0.6931471805599453;
static const double PI_4 = 0.7853981633974483;
static const double SQRT2 = 1.4142135623730951;

static double log_c[11], cos_c[10], sin_c[10];
static int coef_ready = 0;

/* The series coefficients are handed in by the Python definition
 * (1/(2k+1), (-1)^j/(2j)!, (-1)^j/(2j+1)!), so both use the same doubles. */
void pmgen_set_coef(const double* lc, const double* cc, const double* sc) {
  for (int k = 0; k < 11; ++k) log_c[k] = lc[k];
  for (int j = 0; j < 10; ++j) { cos_c[j] = cc[j]; sin_c[j] = sc[j]; }
  coef_ready = 1;
}

static inline double neg2_ln_u(uint32_t h1) {
  double n = (double)h1 * 2.0 + 1.0;
  int ei;
  double m = frexp(n, &ei);
  double e = (double)ei;
  m = m * 2.0;
  e = e - 1.0;
  if (m > SQRT2) { m = m * 0.5; e = e + 1.0; }
  double s = (m - 1.0) / (m + 1.0);
  double t = s * s;
  double acc = t * 0.0 + log_c[10];
  for (int k = 9; k >= 0; --k) acc = acc * t + log_c[k];
  double ln_u = (e - 33.0) * LN2 + 2.0 * s * acc;
  return -2.0 * ln_u;
}

static inline double cos_2pi_u(uint32_t h2) {
  uint32_t q = h2 >> 29;
  double rem = (double)(h2 & 0x1FFFFFFFu) * 2.0 + 1.0;
  double r = rem * (1.0 / 1073741824.0);
  double a = (q & 1u) ? -((1.0 - r) * PI_4) : r * PI_4;
  uint32_t quad = ((q + 1u) >> 1) & 3u;
  double t = a * a;
  double c = t * 0.0 + cos_c[9];
  double sn = t * 0.0 + sin_c[9];
  for (int j = 8; j >= 0; --j) {
    c = c * t + cos_c[j];
    sn = sn * t + sin_c[j];
  }
  sn = sn * a;
  if (quad == 0) return c;
  if (quad == 1) return -sn;
  if (quad == 2) return -c;
  return sn;
}

static inline uint16_t bf16_bits(double x) {
  float f = (float)x;
  union { float f; uint32_t u; } v;
  v.f = f;
  uint32_t b = v.u;
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

void pmgen_words(uint32_t key, uint64_t start, uint64_t count, uint32_t* h1, uint32_t* h2) {
  uint32_t k1 = fmix32(key ^ 0x68E31DA4u), k2 = fmix32(key ^ 0xB5297A4Du);
  for (uint64_t i = 0; i < count; ++i) {
    uint64_t idx = start + i;
    uint32_t lo = (uint32_t)idx, hi = (uint32_t)(idx >> 32);
    if (h1) h1[i] = fmix32(lo ^ fmix32(hi ^ k1));
    if (h2) h2[i] = fmix32(lo ^ fmix32(hi ^ k2));
  }
}

void pmgen_normal_bf16(uint32_t key, uint64_t start, uint64_t count, double mean, double stdv,
                       uint16_t* out) {
  if (!coef_ready) return;
  uint32_t k1 = fmix32(key ^ 0x68E31DA4u), k2 = fmix32(key ^ 0xB5297A4Du);
  for (uint64_t i = 0; i < count; ++i) {
    uint64_t idx = start + i;
    uint32_t lo = (uint32_t)idx, hi = (uint32_t)(idx >> 32);
    uint32_t a = fmix32(lo ^ fmix32(hi ^ k1));
    uint32_t b = fmix32(lo ^ fmix32(hi ^ k2));
    double z = sqrt(neg2_ln_u(a)) * cos_2pi_u(b);
    out[i] = bf16_bits(z * stdv + mean);
  }
}

int pmgen_ready(void) { return coef_ready; }
