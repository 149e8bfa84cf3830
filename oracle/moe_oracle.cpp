// CPU oracle for the quantised MoE FFN layer.  TEST INFRASTRUCTURE ONLY: it is
// used by the tests, by the smoke check and by the CPU-baseline timing, and
// it shares no code with the GPU library.
//
// It is deliberately plain and slow: every weight is decoded from its code
// and scale inside the dot product that uses it, every sum runs in double in
// ascending index order, routing sorts all experts with std::sort, and the
// experts are looped token by token, slot by slot.  OpenMP only splits
// independent output rows, so results are bitwise identical at any thread
// count.
//
// What it computes (the layer the pages describe):
//  * weights are 4-bit: W4A16, INT4 weights with FP16 activations
//    ("GLM-5.3-Flash 320B MoEを4枚のCMP 170HXで動かすvLLMレシピ", 648news.com,
//    section "OpenAI互換APIで動く320BパラメータのMoE構成"); int4 with one scale
//    per row ("Show HN: 低速のコンピュータでGLM 5.2を動かす方法", hakusoku.com,
//    section 実装済み機能); or NVFP4-style e2m1 codes decoded inside the matmul
//    ("GTX 1070向け35BパラメータMoEモデル推論エンジン公開", 648news.com, section
//    "VRAMとシステムメモリで重みを分割する設計" and the NVFP4 glossary entry);
//    or the int8 and int2 per-row-scale formats of the same Colibrì kernels
//    (hakusoku.com, section 実装済み機能);
//  * a DeepSeek-V3-style sigmoid router and a shared expert (hakusoku.com,
//    section 実装済み機能), 8 of 256 experts per token (same page, sections
//    Colibrì and 性能・要件);
//  * the batch-wise expert union: each unique expert of the batch is taken
//    once and applied to every position that chose it (same page, section
//    実装済み機能);
//  * a fixed, deterministic top-k and expert order (648news.com vLLM recipe,
//    section "Ampere世代のGPU向けに最適化された独自カーネル群").
// Readings where the pages are silent (SwiGLU expert, renormalised weights,
// fp64 router, tie-break to the lower index, slot order by descending score,
// optional logit bias, E2M1 tensor scale g) are stated next to the code that
// takes them.
//
// Build: g++ -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

enum { FMT_INT4_ROW = 0, FMT_E2M1_B16 = 1, FMT_INT8_ROW = 2, FMT_INT2_ROW = 3 };

// Bits per stored code of each format.
int code_bits(int fmt) { return fmt == FMT_INT8_ROW ? 8 : fmt == FMT_INT2_ROW ? 2 : 4; }

struct Dims {
  int H, I, E, k, has_shared, fmt;
};

// IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
double fp16_value(uint16_t bits) {
  const int sign = (bits >> 15) & 1;
  const int exp = (bits >> 10) & 0x1F;
  const int frac = bits & 0x3FF;
  double mag;
  if (exp == 0) {
    mag = std::ldexp((double)frac, -24);  // subnormal: frac * 2^-14 / 2^10
  } else if (exp == 31) {
    mag = frac ? NAN : INFINITY;
  } else {
    mag = std::ldexp(1024.0 + frac, exp - 25);  // (1 + frac/2^10) * 2^(exp-15)
  }
  return sign ? -mag : mag;
}

// Element `col` of a nibble-packed row: element 2j is the low nibble of byte j.
inline int nibble(const uint8_t* row, int64_t col) {
  const uint8_t b = row[col >> 1];
  return (col & 1) ? (b >> 4) : (b & 0xF);
}

// Two's-complement int4: codes 8..15 stand for -8..-1.
inline int int4_value(int code) { return code >= 8 ? code - 16 : code; }

// Two's-complement int8: bytes 128..255 stand for -128..-1.
inline int int8_value(uint8_t b) { return b >= 128 ? (int)b - 256 : (int)b; }

// Element `col` of a 2-bit-packed row: element 4j+i sits in bits 2i..2i+1
// of byte j; two's complement, so codes 2 and 3 stand for -2 and -1.
inline int int2_value(const uint8_t* row, int64_t col) {
  const int code = (row[col >> 2] >> (2 * (col & 3))) & 3;
  return code >= 2 ? code - 4 : code;
}

// OCP FP4 E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
// Exponent 0 is subnormal (0 or 0.5); otherwise (1 + m/2) * 2^(e-1).
double e2m1_value(int code) {
  const int sign = (code >> 3) & 1;
  const int e = (code >> 1) & 3;
  const int m = code & 1;
  const double mag = (e == 0) ? 0.5 * m : (1.0 + 0.5 * m) * std::ldexp(1.0, e - 1);
  return sign ? -mag : mag;
}

// OCP FP8 E4M3 ("FN"): bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0
// mantissa; no infinities; exponent 15 with mantissa 7 is NaN.
double e4m3_value(uint8_t b) {
  const int sign = (b >> 7) & 1;
  const int e = (b >> 3) & 0xF;
  const int m = b & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) mag = std::ldexp((double)m, -9);  // (m/8) * 2^-6
  else mag = (1.0 + m / 8.0) * std::ldexp(1.0, e - 7);
  return sign ? -mag : mag;
}

// One quantised matrix in canonical storage: q[rows][cols*bits/8] codes plus
// either a binary16 scale per row (INT4_ROW, INT8_ROW, INT2_ROW) or an e4m3
// scale per 16 columns and an fp32 tensor scale g (E2M1_B16).  The integer
// formats are those of the Colibrì engine's int8/int4/int2 kernels with a
// scale per row ("Show HN: 低速のコンピュータでGLM 5.2を動かす方法",
// hakusoku.com, section 実装済み機能); the bit layout of int8 and int2 is a
// reading (the page gives none): one byte per int8 code, four int2 codes per
// byte from the least significant bits up, both two's complement.
struct QMat {
  const uint8_t* q;
  const void* s;
  double g;
  int rows, cols, fmt;

  // The real-valued weight W[r][c] that the code and its scales stand for.
  double w(int r, int64_t c) const {
    const uint8_t* row = q + (int64_t)r * cols * code_bits(fmt) / 8;
    const uint16_t* s16 = (const uint16_t*)s;
    if (fmt == FMT_INT8_ROW) return (double)int8_value(row[c]) * fp16_value(s16[r]);
    if (fmt == FMT_INT2_ROW) return (double)int2_value(row, c) * fp16_value(s16[r]);
    const int code = nibble(row, c);
    if (fmt == FMT_INT4_ROW) return (double)int4_value(code) * fp16_value(s16[r]);
    const uint8_t* s8 = (const uint8_t*)s + (int64_t)r * (cols / 16);
    return e2m1_value(code) * e4m3_value(s8[c / 16]) * g;
  }
};

struct Expert {
  QMat gate, up, down;
};

// SiLU(v) = v * sigmoid(v).
inline double silu(double v) { return v / (1.0 + std::exp(-v)); }

// One expert applied to one activation vector (SwiGLU FFN, gate first, no
// biases):  h_i = silu(Wg[i].x) * (Wu[i].x);  o_n = Wd[n].h.
void expert_ffn(const Dims& d, const Expert& ex, const double* x, double* hbuf, double* o) {
#pragma omp parallel for schedule(static)
  for (int i = 0; i < d.I; ++i) {
    double g = 0.0, u = 0.0;
    for (int h = 0; h < d.H; ++h) {
      g += ex.gate.w(i, h) * x[h];
      u += ex.up.w(i, h) * x[h];
    }
    hbuf[i] = silu(g) * u;
  }
#pragma omp parallel for schedule(static)
  for (int n = 0; n < d.H; ++n) {
    double acc = 0.0;
    for (int i = 0; i < d.I; ++i) acc += ex.down.w(n, i) * hbuf[i];
    o[n] = acc;
  }
}

// Adaptive expert top-p ("Show HN: 低速のコンピュータでGLM 5.2を動かす方法",
// hakusoku.com, section 実行・チューニングパラメータ: the --topp option, which
// keeps experts until their cumulative weight reaches p).  Reading taken:
// w holds the k renormalised weights of the ranked slots, in slot order;
// keep the shortest prefix whose cumulative weight reaches p, i.e. the
// smallest m with w_0 + ... + w_{m-1} >= p, summed in double in slot
// order.  p is the layer's binary32 parameter, widened exactly.  Returns m
// (k when p <= 0 or p >= 1, or when no prefix reaches p).
int top_p_keep(const double* w, int k, float top_p) {
  if (!(top_p > 0.0f && top_p < 1.0f)) return k;
  const double p = (double)top_p;
  double cum = 0.0;
  for (int j = 0; j < k; ++j) {
    cum += w[j];
    if (cum >= p) return j + 1;
  }
  return k;
}

// Router for one token.  Reading taken: logits in fp64,
// z_e = b_e + sum_h x_h * Wr[e][h] in ascending h; all experts sorted by
// (z descending, expert index ascending) so equal logits go to the lower
// index; the first k are kept in that order; s_j = sigmoid(z_j) and the kept
// weights are renormalised to sum to one, w_j = s_j / sum s.  With adaptive
// top-p only the first m slots are kept (top_p_keep) and renormalised over
// those; slots j >= m get index -1 and weight 0.
void route_token(const Dims& d, const uint16_t* xrow, const float* Wr, const float* b, float top_p,
                 int* idx, double* w, double* z) {
  std::vector<double> xd(d.H);
  for (int h = 0; h < d.H; ++h) xd[h] = fp16_value(xrow[h]);
  for (int e = 0; e < d.E; ++e) {
    double acc = b ? (double)b[e] : 0.0;
    const float* wr = Wr + (int64_t)e * d.H;
    for (int h = 0; h < d.H; ++h) acc += xd[h] * (double)wr[h];
    z[e] = acc;
  }
  std::vector<int> order(d.E);
  for (int e = 0; e < d.E; ++e) order[e] = e;
  std::sort(order.begin(), order.end(), [&](int a, int c) {
    if (z[a] != z[c]) return z[a] > z[c];
    return a < c;
  });
  // sigmoid scores of the k ranked slots, renormalised to sum to one
  std::vector<double> s(d.k), wk(d.k);
  double ssum = 0.0;
  for (int j = 0; j < d.k; ++j) {
    s[j] = 1.0 / (1.0 + std::exp(-z[order[j]]));
    ssum += s[j];
  }
  for (int j = 0; j < d.k; ++j) wk[j] = s[j] / ssum;
  // adaptive top-p keeps the first m slots; their weights are renormalised
  // over the kept slots
  const int m = top_p_keep(wk.data(), d.k, top_p);
  double msum = 0.0;
  for (int j = 0; j < m; ++j) msum += s[j];
  for (int j = 0; j < m; ++j) {
    idx[j] = order[j];
    w[j] = s[j] / msum;
  }
  for (int j = m; j < d.k; ++j) {
    idx[j] = -1;
    w[j] = 0.0;
  }
}

bool dims_ok(const Dims& d) {
  return d.H > 0 && d.I > 0 && d.E > 0 && d.k >= 1 && d.k <= d.E && d.H % 32 == 0 && d.I % 32 == 0 &&
         d.fmt >= FMT_INT4_ROW && d.fmt <= FMT_INT2_ROW;
}

Dims to_dims(const int32_t* p) { return Dims{p[0], p[1], p[2], p[3], p[4], p[5]}; }

}  // namespace

extern "C" {

// ---- code tables, exposed so the tests can pin them ----------------------
void oracle_fp16_values(const uint16_t* in, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = fp16_value(in[i]);
}
// Two codes per byte, even element from the low nibble.
void oracle_int4_values(const uint8_t* q, int64_t nbytes, int32_t* out) {
  for (int64_t i = 0; i < 2 * nbytes; ++i) out[i] = int4_value(nibble(q, i));
}
void oracle_int8_values(const uint8_t* q, int64_t nbytes, int32_t* out) {
  for (int64_t i = 0; i < nbytes; ++i) out[i] = int8_value(q[i]);
}
// Four codes per byte, element 4j+i from bits 2i..2i+1 of byte j.
void oracle_int2_values(const uint8_t* q, int64_t nbytes, int32_t* out) {
  for (int64_t i = 0; i < 4 * nbytes; ++i) out[i] = int2_value(q, i);
}
void oracle_e2m1_values(const uint8_t* q, int64_t nbytes, double* out) {
  for (int64_t i = 0; i < 2 * nbytes; ++i) out[i] = e2m1_value(nibble(q, i));
}
void oracle_e4m3_values(const uint8_t* s, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_value(s[i]);
}

// Dense weight matrix W[rows][cols] (double) of one canonical matrix.
int oracle_dequant(int32_t fmt, const uint8_t* q, const void* s, float g, int32_t rows, int32_t cols,
                   double* out) {
  if (cols % 32 || rows <= 0 || fmt < FMT_INT4_ROW || fmt > FMT_INT2_ROW) return -1;
  QMat m{q, s, (double)g, rows, cols, fmt};
  for (int r = 0; r < rows; ++r)
    for (int c = 0; c < cols; ++c) out[(int64_t)r * cols + c] = m.w(r, c);
  return 0;
}

// Routing and the batch union.
//   dims: int32[6] = {H, I, E, k, has_shared, fmt}
//   x: binary16 bits [T][H]; Wr: fp32 [E][H]; b: fp32 [E] or NULL
//   top_p: adaptive top-p threshold, the layer's binary32 parameter (0 keeps
//   all k slots)
//   outputs: topk_idx int32 [T][k], topk_w fp32 [T][k], z fp64 [T][E] (nullable),
//   n_unique int32[1], uniq_ids int32[min(E,T*k)], uniq_off int32[min(E,T*k)+1],
//   pairs int32[T*k] (pair id t*k+j of the kept slots, grouped by expert
//   ascending, tokens ascending; uniq_off[n_unique] = number of kept pairs).
int oracle_route(const int32_t* dims, float top_p, const uint16_t* x, int32_t T, const float* Wr, const float* b,
                 int32_t* topk_idx, float* topk_w, double* z_out, int32_t* n_unique, int32_t* uniq_ids,
                 int32_t* uniq_off, int32_t* pairs) {
  const Dims d = to_dims(dims);
  if (!dims_ok(d) || T < 0) return -1;
  std::vector<int> idx((size_t)T * d.k);
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    std::vector<double> z(d.E), w(d.k);
    route_token(d, x + (int64_t)t * d.H, Wr, b, top_p, &idx[(size_t)t * d.k], w.data(), z.data());
    for (int j = 0; j < d.k; ++j) {
      topk_idx[(int64_t)t * d.k + j] = idx[(size_t)t * d.k + j];
      topk_w[(int64_t)t * d.k + j] = (float)w[j];
    }
    if (z_out) std::memcpy(z_out + (int64_t)t * d.E, z.data(), sizeof(double) * d.E);
  }
  // Union: experts chosen by any token, ascending; for each, its (token,
  // slot) pairs in ascending token order.  Brute force over all pairs.
  int nu = 0, np = 0;
  for (int e = 0; e < d.E; ++e) {
    int start = np;
    for (int t = 0; t < T; ++t)
      for (int j = 0; j < d.k; ++j)
        if (idx[(size_t)t * d.k + j] == e) pairs[np++] = t * d.k + j;
    if (np > start) {
      uniq_ids[nu] = e;
      uniq_off[nu] = start;
      ++nu;
    }
  }
  uniq_off[nu] = np;
  *n_unique = nu;
  return 0;
}

// The whole layer for the tokens in token_list (all T tokens when NULL):
// y[t] = sum_j w_j * FFN_{e_j}(x_t) + FFN_shared(x_t), accumulated in double
// in slot order over the kept slots, shared expert last, with weight one.
//   experts: arrays of E(+1) host pointers per canonical tensor; index E is
//   the shared expert.  Unselected experts may be NULL.  g3: fp32 [E+1][3]
//   tensor scales (gate, up, down), or NULL meaning 1.0.
//   y: fp64 [n_list][H].  Returns 0, or -1 on bad arguments, -2 when a
//   selected expert pointer is NULL.
int oracle_forward(const int32_t* dims, float top_p, const void* const* qg, const void* const* sg, const void* const* qu,
                   const void* const* su, const void* const* qd, const void* const* sd, const float* g3,
                   const float* Wr, const float* b, const uint16_t* x, int32_t T, const int32_t* token_list,
                   int32_t n_list, double* y, int32_t n_threads) {
  const Dims d = to_dims(dims);
  if (!dims_ok(d) || T < 0) return -1;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#endif
  const int n = token_list ? n_list : T;
  auto expert_at = [&](int e) {
    auto G = [&](int m) { return g3 ? (double)g3[(int64_t)e * 3 + m] : 1.0; };
    Expert ex;
    ex.gate = QMat{(const uint8_t*)qg[e], sg[e], G(0), d.I, d.H, d.fmt};
    ex.up = QMat{(const uint8_t*)qu[e], su[e], G(1), d.I, d.H, d.fmt};
    ex.down = QMat{(const uint8_t*)qd[e], sd[e], G(2), d.H, d.I, d.fmt};
    return ex;
  };
  auto present = [&](int e) { return qg[e] && sg[e] && qu[e] && su[e] && qd[e] && sd[e]; };
  std::vector<double> xd(d.H), hbuf(d.I), o(d.H), z(d.E), w(d.k);
  std::vector<int> idx(d.k);
  for (int ti = 0; ti < n; ++ti) {
    const int t = token_list ? token_list[ti] : ti;
    if (t < 0 || t >= T) return -1;
    const uint16_t* xrow = x + (int64_t)t * d.H;
    for (int h = 0; h < d.H; ++h) xd[h] = fp16_value(xrow[h]);
    route_token(d, xrow, Wr, b, top_p, idx.data(), w.data(), z.data());
    double* yt = y + (int64_t)ti * d.H;
    for (int c = 0; c < d.H; ++c) yt[c] = 0.0;
    for (int j = 0; j < d.k; ++j) {
      if (idx[j] < 0) continue;  // slot dropped by adaptive top-p
      if (!present(idx[j])) return -2;
      expert_ffn(d, expert_at(idx[j]), xd.data(), hbuf.data(), o.data());
      for (int c = 0; c < d.H; ++c) yt[c] += w[j] * o[c];
    }
    if (d.has_shared) {
      if (!present(d.E)) return -2;
      expert_ffn(d, expert_at(d.E), xd.data(), hbuf.data(), o.data());
      for (int c = 0; c < d.H; ++c) yt[c] += o[c];
    }
  }
  return 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

}  // extern "C"
