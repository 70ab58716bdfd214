/*
 * cam_oracle.c -- plain, slow, obviously correct CPU oracle for the per-GPU hot
 * path of sequence/context-parallel attention movement.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg load it.  It shares no code, header, table or helper with the
 * HIP path.
 *
 * Sources (web pages, cited by title and section):
 *  [FV]  FastVideo compare view "[perf] Probe H3 chunked all-to-all with direct
 *        output slices": the Ulysses all_to_all_4D relayout (scatter dim 2 /
 *        gather dim 1 and the inverse), benchmark_ulysses_a2a.py operand shapes.
 *  [VA]  vllm-ascend PR "[Performance][Attention] Fuse local SFA LSE formation
 *        into DCP pack": "What this PR does" (LSE = softmax_max +
 *        log(softmax_sum), invalid statistics give -inf, stable combine) and
 *        "How was this patch tested?" (special cases).
 *  [CU]  cuLA PR "feat(distributed): add packed hybrid runtime and THD
 *        planner": packed THD cu_seqlens, logical CP ranks in one process.
 *
 * Training: the relayout's gradient is its inverse relayout ([FV] benchmark's
 * forward/backward pair, whose gradients must equal the collective's), and the
 * combine's gradient is its derivative, written out below ([CU] forward and
 * backward comparison of context parallelism; the pages print no formula).
 *
 * Arithmetic: every floating-point result is computed in double and rounded
 * once at the end (bf16 / fp16 round-to-nearest-even, fp32 by the C cast),
 * since the pages do not fix the precision of the reduction.
 *
 * Readings of points the pages leave open are marked "reading:".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Number formats (IEEE 754 binary16 and the bfloat16 truncation of binary32) */
/* ------------------------------------------------------------------------ */

/* Round a double to a binary format with `prec` significand bits (implicit bit
 * included), smallest normal exponent `emin` and largest exponent `emax`,
 * round-to-nearest, ties to even; returns the rounded value as a double
 * (exactly representable in that format) or +-inf on overflow. */
static double round_to_format(double x, int prec, int emin, int emax)
{
    if (isnan(x) || isinf(x) || x == 0.0)
        return x;
    int e;
    frexp(fabs(x), &e);           /* |x| in [2^(e-1), 2^e) */
    int ex = e - 1;
    if (ex < emin)
        ex = emin;                /* subnormal range: fixed spacing */
    double spacing = ldexp(1.0, ex - (prec - 1));
    double q = nearbyint(x / spacing); /* x / spacing is exact (power of two) */
    double y = q * spacing;
    double maxfinite = ldexp(2.0 - ldexp(1.0, -(prec - 1)), emax);
    if (fabs(y) > maxfinite)
        return copysign(INFINITY, x);
    return y;
}

uint16_t orc_double_to_bf16(double x)
{
    if (isnan(x))
        return (uint16_t)(signbit(x) ? 0xFFC0u : 0x7FC0u);
    double y = round_to_format(x, 8, -126, 127);
    float f = (float)y;           /* exact: y has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

double orc_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

uint16_t orc_double_to_fp16(double x)
{
    if (isnan(x))
        return (uint16_t)(signbit(x) ? 0xFE00u : 0x7E00u);
    double y = round_to_format(x, 11, -14, 15);
    uint16_t sign = signbit(y) ? 0x8000u : 0u;
    double a = fabs(y);
    if (isinf(a))
        return sign | 0x7C00u;
    if (a == 0.0)
        return sign;
    if (a < ldexp(1.0, -14))      /* subnormal: a = m * 2^-24 */
        return sign | (uint16_t)(a / ldexp(1.0, -24));
    int e;
    frexp(a, &e);
    int ex = e - 1;               /* a in [2^ex, 2^(ex+1)) */
    double frac = a / ldexp(1.0, ex) - 1.0;
    return sign | (uint16_t)((ex + 15) << 10) | (uint16_t)(frac * 1024.0);
}

double orc_fp16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1F;
    int man = h & 0x3FF;
    double v;
    if (ex == 0)
        v = ldexp((double)man, -24);
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp(1.0 + man / 1024.0, ex - 15);
    return sign ? -v : v;
}

/* dtype codes: 0 = bf16, 1 = fp16 (16-bit storage, double arithmetic). */
static double load_half(const void* base, int64_t elem_index, int dtype)
{
    uint16_t b;
    memcpy(&b, (const char*)base + 2 * elem_index, 2);
    return dtype == 0 ? orc_bf16_to_double(b) : orc_fp16_to_double(b);
}

static void store_half(void* base, int64_t elem_index, int dtype, double v)
{
    uint16_t b = dtype == 0 ? orc_double_to_bf16(v) : orc_double_to_fp16(v);
    memcpy((char*)base + 2 * elem_index, &b, 2);
}

void orc_round_bf16_array(const double* x, uint16_t* y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        y[i] = orc_double_to_bf16(x[i]);
}

void orc_round_fp16_array(const double* x, uint16_t* y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        y[i] = orc_double_to_fp16(x[i]);
}

void orc_bf16_to_double_array(const uint16_t* x, double* y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        y[i] = orc_bf16_to_double(x[i]);
}

void orc_fp16_to_double_array(const uint16_t* x, double* y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        y[i] = orc_fp16_to_double(x[i]);
}

/* ------------------------------------------------------------------------ */
/* Dense Ulysses relayout  ([FV], ulysses_a2a.py and benchmark_ulysses_a2a.py) */
/* ------------------------------------------------------------------------ */
/*
 * P logical ranks live in one buffer, rank outermost (reading: the stack order
 * of the emulated ranks is [P] then the B batch planes, B = 3 carrying Q, K, V).
 *
 * Sequence-sharded side: in[j][b][s][h][d], rank j holds tokens
 *   [j*S/P, (j+1)*S/P) of every plane, all H heads.
 * Head-sharded side:     out[r][b][t][h'][d], rank r holds heads
 *   [r*H/P, (r+1)*H/P) (reading: contiguous head blocks, sequence blocks
 *   concatenated in source-rank order), all S tokens.
 *
 * seq->head (all_to_all_4D scatter dim 2, gather dim 1):
 *   out[r][b][j*S/P + s][h][d] = in[j][b][s][r*H/P + h][d]
 * head->seq (scatter dim 1, gather dim 2) is the inverse map.
 * Elements are `esize` bytes and are copied as bits.
 */
void orc_seq_to_head(const void* in, void* out, int64_t P, int64_t B, int64_t S,
                     int64_t H, int64_t D, int64_t esize)
{
    const char* src = (const char*)in;
    char* dst = (char*)out;
    int64_t Sp = S / P, Hp = H / P;
    for (int64_t r = 0; r < P; ++r)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t j = 0; j < P; ++j)
                for (int64_t s = 0; s < Sp; ++s)
                    for (int64_t h = 0; h < Hp; ++h) {
                        int64_t o = (((r * B + b) * S + j * Sp + s) * Hp + h) * D;
                        int64_t i = (((j * B + b) * Sp + s) * H + r * Hp + h) * D;
                        memcpy(dst + o * esize, src + i * esize, (size_t)(D * esize));
                    }
}

void orc_head_to_seq(const void* in, void* out, int64_t P, int64_t B, int64_t S,
                     int64_t H, int64_t D, int64_t esize)
{
    const char* src = (const char*)in;
    char* dst = (char*)out;
    int64_t Sp = S / P, Hp = H / P;
    for (int64_t j = 0; j < P; ++j)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t s = 0; s < Sp; ++s)
                for (int64_t r = 0; r < P; ++r)
                    for (int64_t h = 0; h < Hp; ++h) {
                        int64_t o = (((j * B + b) * Sp + s) * H + r * Hp + h) * D;
                        int64_t i = (((r * B + b) * S + j * Sp + s) * Hp + h) * D;
                        memcpy(dst + o * esize, src + i * esize, (size_t)(D * esize));
                    }
}

/* ------------------------------------------------------------------------ */
/* Varlen (packed THD, cu_seqlens) relayout  ([CU] description and review notes
 * on cu_seqlens shard offsets; [FV] relayout per token)                     */
/* ------------------------------------------------------------------------ */
/*
 * Reading: sequence i = tokens [cu[i], cu[i+1]) of length L is cut into P
 * pieces, piece p = in-sequence positions [floor(p*L/P), floor((p+1)*L/P)),
 * and piece p lives on logical rank p.  Rank p stores its pieces in sequence
 * order: its token count is T_p = sum_i |piece_p(i)|, its slab [B][T_p][H][D]
 * starts at token offset R_p = T_0 + ... + T_{p-1} of a [B]-planed rank-major
 * buffer (element offset B*R_p*H*D).  With one sequence and P | T this is the
 * dense layout above.
 */
static int64_t piece_start(int64_t p, int64_t L, int64_t P) { return (p * L) / P; }

/* Host plan: rank_cu[p*(nseq+1) + i] = tokens of rank p that precede sequence
 * i; rank_off[p] = R_p (rank_off[P] = total).  Written as plain counting. */
void orc_varlen_plan(const int32_t* cu, int64_t nseq, int64_t P, int32_t* rank_cu,
                     int64_t* rank_off)
{
    int64_t off = 0;
    for (int64_t p = 0; p < P; ++p) {
        rank_off[p] = off;
        int64_t acc = 0;
        for (int64_t i = 0; i < nseq; ++i) {
            rank_cu[p * (nseq + 1) + i] = (int32_t)acc;
            int64_t L = (int64_t)cu[i + 1] - cu[i];
            acc += piece_start(p + 1, L, P) - piece_start(p, L, P);
        }
        rank_cu[p * (nseq + 1) + nseq] = (int32_t)acc;
        off += acc;
    }
    rank_off[P] = off;
}

/* direction 0: seq->head (in rank-major ragged, out [P][B][T][H/P][D]);
 * direction 1: head->seq (the inverse). */
static void varlen_relayout(const void* in, void* out, const int32_t* cu, int64_t nseq,
                            int64_t P, int64_t B, int64_t H, int64_t D, int64_t esize,
                            int direction)
{
    const char* src = (const char*)in;
    char* dst = (char*)out;
    int64_t T = cu[nseq];
    int64_t Hp = H / P;
    int64_t R = 0; /* token offset of rank p's slab */
    for (int64_t p = 0; p < P; ++p) {
        int64_t Tp = 0;
        for (int64_t i = 0; i < nseq; ++i) {
            int64_t L = (int64_t)cu[i + 1] - cu[i];
            Tp += piece_start(p + 1, L, P) - piece_start(p, L, P);
        }
        for (int64_t b = 0; b < B; ++b) {
            int64_t l = 0; /* local row on rank p */
            for (int64_t i = 0; i < nseq; ++i) {
                int64_t L = (int64_t)cu[i + 1] - cu[i];
                for (int64_t k = piece_start(p, L, P); k < piece_start(p + 1, L, P); ++k) {
                    int64_t t = cu[i] + k;
                    for (int64_t r = 0; r < P; ++r)
                        for (int64_t h = 0; h < Hp; ++h) {
                            int64_t seq_side = ((B * R + b * Tp + l) * H + r * Hp + h) * D;
                            int64_t head_side = (((r * B + b) * T + t) * Hp + h) * D;
                            if (direction == 0)
                                memcpy(dst + head_side * esize, src + seq_side * esize,
                                       (size_t)(D * esize));
                            else
                                memcpy(dst + seq_side * esize, src + head_side * esize,
                                       (size_t)(D * esize));
                        }
                    ++l;
                }
            }
        }
        R += Tp;
    }
}

void orc_varlen_seq_to_head(const void* in, void* out, const int32_t* cu, int64_t nseq,
                            int64_t P, int64_t B, int64_t H, int64_t D, int64_t esize)
{
    varlen_relayout(in, out, cu, nseq, P, B, H, D, esize, 0);
}

void orc_varlen_head_to_seq(const void* in, void* out, const int32_t* cu, int64_t nseq,
                            int64_t P, int64_t B, int64_t H, int64_t D, int64_t esize)
{
    varlen_relayout(in, out, cu, nseq, P, B, H, D, esize, 1);
}

/* ------------------------------------------------------------------------ */
/* LSE formation and the max/sum-aware pack  ([VA] "What this PR does")       */
/* ------------------------------------------------------------------------ */
/* LSE = softmax_max + log(softmax_sum); a non-finite max, a non-finite sum or a
 * sum <= 0 is an invalid contribution, written as -inf (natural log; -0.0 and
 * NaN sums are invalid because they fail "> 0"). */
double orc_lse_from_stats(float m, float s)
{
    if (isfinite(m) && isfinite(s) && s > 0.0f)
        return (double)m + log((double)s);
    return -INFINITY;
}

/* Packed exchange layout (reading: the pages say the mapping of rows, heads
 * and tokens and the meaning of the packed payload stay as they were, but
 * print no byte layout).  For source rank p and
 * destination rank r, chunk (p, r) holds the rows rank r will combine:
 *   scatter_dim = 1 (heads):  rows (t, h') for t < T, h' < H/P, source head
 *                             r*H/P + h'; row index q = t*(H/P) + h'.
 *   scatter_dim = 0 (tokens): rows (t', h) for t' < T/P, h < H, source token
 *                             r*T/P + t'; row index q = t'*H + h.
 * A chunk is the O-region [rows][Dv] in the payload dtype, padded to 16 bytes,
 * then the L-region [rows] fp32, padded to 16 bytes.  Chunks are stored
 * [P_src][P_dst].  Padding bytes carry no payload. */
static int64_t round16(int64_t x) { return (x + 15) / 16 * 16; }

int64_t orc_pack_rows(int64_t P, int64_t T, int64_t H, int scatter_dim)
{
    return scatter_dim == 1 ? T * (H / P) : (T / P) * H;
}

int64_t orc_pack_chunk_bytes(int64_t P, int64_t T, int64_t H, int64_t Dv, int scatter_dim,
                             int64_t esize)
{
    int64_t rows = orc_pack_rows(P, T, H, scatter_dim);
    return round16(rows * Dv * esize) + round16(rows * 4);
}

/* Strides are in elements; Dv is contiguous. */
void orc_lse_pack(const void* out, int64_t o_sp, int64_t o_st, int64_t o_sh,
                  const float* smax, int64_t m_sp, int64_t m_st, int64_t m_sh,
                  const float* ssum, int64_t s_sp, int64_t s_st, int64_t s_sh,
                  int64_t P, int64_t T, int64_t H, int64_t Dv, int scatter_dim,
                  int64_t esize, void* packed)
{
    const char* src = (const char*)out;
    char* dst = (char*)packed;
    int64_t rows = orc_pack_rows(P, T, H, scatter_dim);
    int64_t o_bytes = round16(rows * Dv * esize);
    int64_t chunk = orc_pack_chunk_bytes(P, T, H, Dv, scatter_dim, esize);
    for (int64_t p = 0; p < P; ++p)
        for (int64_t r = 0; r < P; ++r) {
            char* obase = dst + (p * P + r) * chunk;
            float* lbase = (float*)(obase + o_bytes);
            for (int64_t q = 0; q < rows; ++q) {
                int64_t t, h;
                if (scatter_dim == 1) {
                    t = q / (H / P);
                    h = r * (H / P) + q % (H / P);
                } else {
                    t = r * (T / P) + q / H;
                    h = q % H;
                }
                memcpy(obase + q * Dv * esize, src + (p * o_sp + t * o_st + h * o_sh) * esize,
                       (size_t)(Dv * esize));
                float m = smax[p * m_sp + t * m_st + h * m_sh];
                float s = ssum[p * s_sp + t * s_st + h * s_sh];
                lbase[q] = (float)orc_lse_from_stats(m, s);
            }
        }
}

/* ------------------------------------------------------------------------ */
/* Stable LSE-weighted combine  ([VA] "What this PR does": kept unchanged)    */
/* ------------------------------------------------------------------------ */
/*
 * For one output row: V = {p : L_p finite}; M = max_{p in V} L_p;
 * w_p = exp(L_p - M); Z = sum w_p; out = sum_{p in V} w_p O_p / Z;
 * lse_out = M + log Z.  Reading: an empty V gives out = +0 and lse_out = -inf,
 * and an invalid partial's O row is never read (so it may hold anything).
 * Partials are visited in ascending p.
 *
 * part_o[p*D + d] and part_l[p] for one row, valid[p] gates each partial.
 */
void orc_combine_row_f64(const double* part_o, const double* part_l, const int* valid,
                         int64_t P, int64_t D, double* out, double* lse_out)
{
    double M = -INFINITY;
    int any = 0;
    for (int64_t p = 0; p < P; ++p)
        if (valid[p] && isfinite(part_l[p])) {
            if (!any || part_l[p] > M)
                M = part_l[p];
            any = 1;
        }
    if (!any) {
        for (int64_t d = 0; d < D; ++d)
            out[d] = 0.0;
        *lse_out = -INFINITY;
        return;
    }
    double Z = 0.0;
    for (int64_t d = 0; d < D; ++d)
        out[d] = 0.0;
    for (int64_t p = 0; p < P; ++p) {
        if (!(valid[p] && isfinite(part_l[p])))
            continue;
        double w = exp(part_l[p] - M);
        Z += w;
        for (int64_t d = 0; d < D; ++d)
            out[d] += w * part_o[p * D + d];
    }
    for (int64_t d = 0; d < D; ++d)
        out[d] /= Z;
    *lse_out = M + log(Z);
}

/* Dense double combine: part_o [P][R][D], part_l [P][R] -> out [R][D], lse [R]. */
void orc_combine_f64(const double* part_o, const double* part_l, int64_t P, int64_t R,
                     int64_t D, double* out, double* lse)
{
    double* po = (double*)malloc(sizeof(double) * (size_t)(P * D + 1));
    double* pl = (double*)malloc(sizeof(double) * (size_t)(P + 1));
    int* valid = (int*)malloc(sizeof(int) * (size_t)(P + 1));
    for (int64_t row = 0; row < R; ++row) {
        for (int64_t p = 0; p < P; ++p) {
            pl[p] = part_l[p * R + row];
            valid[p] = 1;
            for (int64_t d = 0; d < D; ++d)
                po[p * D + d] = part_o[(p * R + row) * D + d];
        }
        orc_combine_row_f64(po, pl, valid, P, D, out + row * D, lse + row);
    }
    free(po);
    free(pl);
    free(valid);
}

/* Causal validity of KV piece p for token t of a packed THD batch (reading:
 * partial p of token (i, k) is the attention of that query over piece p of its
 * own sequence under a causal mask; it has at least one visible key, and is
 * therefore valid, iff piece p is non-empty and starts at or before k). */
int orc_causal_piece_valid(const int32_t* cu, int64_t nseq, int64_t P, int64_t p, int64_t t)
{
    for (int64_t i = 0; i < nseq; ++i) {
        if (t >= cu[i] && t < cu[i + 1]) {
            int64_t L = (int64_t)cu[i + 1] - cu[i];
            int64_t k = t - cu[i];
            int64_t a = piece_start(p, L, P), e = piece_start(p + 1, L, P);
            return a < e && a <= k;
        }
    }
    return 0;
}

/*
 * Generic strided combine of P partials over rows (t, h), t in [t_begin, t_end):
 *   part_out  element (p, t, h, d) at po_sp*p + po_st*(t - t_begin) + po_sh*h + d
 *   part_lse  element (p, t, h)    at pl_sp*p + pl_st*(t - t_begin) + pl_sh*h
 *   out       element (t, h, d)    at o_st*(t - t_begin) + o_sh*h + d
 *   lse_out   (nullable)           at lo_st*(t - t_begin) + lo_sh*h
 * (all strides in elements; the pointers address row t_begin, so a sample of
 * rows can be passed without the rest).  With cu_seqlens non-null, partial p of
 * row t is additionally gated by orc_causal_piece_valid (nseq sequences, the
 * P partials being the P KV pieces of each sequence) and is not read when
 * masked.  dtype 0 = bf16, 1 = fp16.
 */
void orc_lse_combine(const void* part_out, int64_t po_sp, int64_t po_st, int64_t po_sh,
                     const float* part_lse, int64_t pl_sp, int64_t pl_st, int64_t pl_sh,
                     int64_t P, int64_t t_begin, int64_t t_end, int64_t H, int64_t D,
                     int dtype, void* out, int64_t o_st, int64_t o_sh, float* lse_out,
                     int64_t lo_st, int64_t lo_sh, const int32_t* cu_seqlens, int64_t nseq)
{
    double* po = (double*)malloc(sizeof(double) * (size_t)(P * D + 1));
    double* pl = (double*)malloc(sizeof(double) * (size_t)(P + 1));
    int* valid = (int*)malloc(sizeof(int) * (size_t)(P + 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)(D + 1));
    for (int64_t t = t_begin; t < t_end; ++t)
        for (int64_t h = 0; h < H; ++h) {
            int64_t tr = t - t_begin;
            for (int64_t p = 0; p < P; ++p) {
                valid[p] = cu_seqlens ? orc_causal_piece_valid(cu_seqlens, nseq, P, p, t) : 1;
                pl[p] = -INFINITY;
                if (!valid[p])
                    continue;
                pl[p] = (double)part_lse[p * pl_sp + tr * pl_st + h * pl_sh];
                if (!isfinite(pl[p]))
                    continue;
                for (int64_t d = 0; d < D; ++d)
                    po[p * D + d] = load_half(part_out, p * po_sp + tr * po_st + h * po_sh + d, dtype);
            }
            double lse;
            orc_combine_row_f64(po, pl, valid, P, D, acc, &lse);
            for (int64_t d = 0; d < D; ++d)
                store_half(out, tr * o_st + h * o_sh + d, dtype, acc[d]);
            if (lse_out)
                lse_out[tr * lo_st + h * lo_sh] = (float)lse;
        }
    free(po);
    free(pl);
    free(valid);
    free(acc);
}

/*
 * Combine over the emulated exchange: destination rank r receives chunk
 * (p, r) from every source p (the all-to-all is a view of the packed buffer,
 * no bytes move).  out row r*rows + q and lse_out (nullable) row r*rows + q,
 * rows as in the pack; Dv contiguous.  For scatter_dim = 1 this is
 * [P_dst][T][H/P][Dv]; for scatter_dim = 0 it is [T][H][Dv].
 */
void orc_lse_combine_packed(const void* packed, int64_t P, int64_t T, int64_t H, int64_t Dv,
                            int scatter_dim, int dtype, void* out, float* lse_out)
{
    const char* src = (const char*)packed;
    int64_t rows = orc_pack_rows(P, T, H, scatter_dim);
    int64_t o_bytes = round16(rows * Dv * 2);
    int64_t chunk = orc_pack_chunk_bytes(P, T, H, Dv, scatter_dim, 2);
    double* po = (double*)malloc(sizeof(double) * (size_t)(P * Dv + 1));
    double* pl = (double*)malloc(sizeof(double) * (size_t)(P + 1));
    int* valid = (int*)malloc(sizeof(int) * (size_t)(P + 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)(Dv + 1));
    for (int64_t r = 0; r < P; ++r)
        for (int64_t q = 0; q < rows; ++q) {
            for (int64_t p = 0; p < P; ++p) {
                const char* c = src + (p * P + r) * chunk;
                float l;
                memcpy(&l, c + o_bytes + 4 * q, 4);
                pl[p] = (double)l;
                valid[p] = 1;
                if (!isfinite(pl[p]))
                    continue;
                for (int64_t d = 0; d < Dv; ++d)
                    po[p * Dv + d] = load_half(c, q * Dv + d, dtype);
            }
            double lse;
            orc_combine_row_f64(po, pl, valid, P, Dv, acc, &lse);
            for (int64_t d = 0; d < Dv; ++d)
                store_half(out, (r * rows + q) * Dv + d, dtype, acc[d]);
            if (lse_out)
                lse_out[r * rows + q] = (float)lse;
        }
    free(po);
    free(pl);
    free(valid);
    free(acc);
}

/* ------------------------------------------------------------------------ */
/* Brute-force attention (tiny end-to-end check; produces partials)           */
/* ------------------------------------------------------------------------ */
/*
 * q, k, v: [T][H][D] in bf16 (dtype 0) or fp16 (dtype 1).  For every query t
 * and head h, attends the keys j in [kv_begin, kv_end) (and j <= t if causal):
 *   score_j = (q_t . k_j) / sqrt(D)        (reading: softmax scale 1/sqrt(D))
 *   softmax_max = max_j score_j,  softmax_sum = sum_j exp(score_j - max),
 *   out = sum_j exp(score_j - max) v_j / softmax_sum.
 * With no visible key: max = -inf, sum = 0, out = 0.  Outputs are double.
 */
void orc_attention(const void* q, const void* k, const void* v, int64_t T, int64_t H,
                   int64_t D, int dtype, int64_t kv_begin, int64_t kv_end, int causal,
                   double* out, double* smax, double* ssum)
{
    double scale = 1.0 / sqrt((double)D);
    double* score = (double*)malloc(sizeof(double) * (size_t)(kv_end - kv_begin + 1));
    for (int64_t t = 0; t < T; ++t)
        for (int64_t h = 0; h < H; ++h) {
            int64_t hi = kv_end;
            if (causal && hi > t + 1)
                hi = t + 1;
            double m = -INFINITY;
            for (int64_t j = kv_begin; j < hi; ++j) {
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    dot += load_half(q, (t * H + h) * D + d, dtype) *
                           load_half(k, (j * H + h) * D + d, dtype);
                score[j - kv_begin] = dot * scale;
                if (score[j - kv_begin] > m)
                    m = score[j - kv_begin];
            }
            double* o = out + (t * H + h) * D;
            for (int64_t d = 0; d < D; ++d)
                o[d] = 0.0;
            double sum = 0.0;
            for (int64_t j = kv_begin; j < hi; ++j) {
                double e = exp(score[j - kv_begin] - m);
                sum += e;
                for (int64_t d = 0; d < D; ++d)
                    o[d] += e * load_half(v, (j * H + h) * D + d, dtype);
            }
            if (sum > 0.0)
                for (int64_t d = 0; d < D; ++d)
                    o[d] /= sum;
            smax[t * H + h] = m;
            ssum[t * H + h] = sum;
        }
    free(score);
}

/* ------------------------------------------------------------------------ */
/* Combine with the sequence-sharded output layout (the combine followed by   */
/* the head->seq relayout of its result, [FV] "direct output slices")         */
/* ------------------------------------------------------------------------ */

/* Rank-major (sequence-sharded) row of every global token of a packed THD
 * batch: token cu[i] + k at position k of piece p of sequence i sits at row
 * R_p + (tokens of rank p before sequence i) + (k - floor(p*L/P)), the order
 * of the varlen relayout's sequence side.  row[t] for t < cu[nseq]. */
void orc_varlen_token_rows(const int32_t* cu, int64_t nseq, int64_t P, int64_t* row)
{
    int64_t R = 0;
    for (int64_t p = 0; p < P; ++p) {
        int64_t l = 0;
        for (int64_t i = 0; i < nseq; ++i) {
            int64_t L = (int64_t)cu[i + 1] - cu[i];
            for (int64_t k = piece_start(p, L, P); k < piece_start(p + 1, L, P); ++k)
                row[cu[i] + k] = R + l++;
        }
        R += l;
    }
}

/* The packed combine, then its result moved to token-major order:
 * out [T][H][Dv], lse_out [T][H] (nullable).  For scatter_dim = 1 the
 * destination-major result row (r, t*(H/P) + h') goes to (t, r*H/P + h');
 * for scatter_dim = 0 the two orders coincide. */
void orc_lse_combine_packed_seq(const void* packed, int64_t P, int64_t T, int64_t H, int64_t Dv,
                                int scatter_dim, int dtype, void* out, float* lse_out)
{
    int64_t rows = orc_pack_rows(P, T, H, scatter_dim);
    uint16_t* tmp = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(P * rows * Dv + 1));
    float* ltmp = (float*)malloc(sizeof(float) * (size_t)(P * rows + 1));
    orc_lse_combine_packed(packed, P, T, H, Dv, scatter_dim, dtype, tmp, ltmp);
    for (int64_t r = 0; r < P; ++r)
        for (int64_t q = 0; q < rows; ++q) {
            int64_t t, h;
            if (scatter_dim == 1) {
                t = q / (H / P);
                h = r * (H / P) + q % (H / P);
            } else {
                t = r * (T / P) + q / H;
                h = q % H;
            }
            memcpy((char*)out + (t * H + h) * Dv * 2, tmp + (r * rows + q) * Dv, (size_t)(Dv * 2));
            if (lse_out)
                lse_out[t * H + h] = ltmp[r * rows + q];
        }
    free(tmp);
    free(ltmp);
}

/* ------------------------------------------------------------------------ */
/* Gradient of the stable combine (training use of the combine)            */
/* ------------------------------------------------------------------------ */
/*
 * Within V the combine of one row is a smooth function of the partials: with
 * lse = log sum_{q in V} exp(L_q) and w_p = exp(L_p - lse),
 *   out = sum_{p in V} w_p O_p,  d out / d O_p = w_p I,
 *   d w_q / d L_p = w_q (delta_pq - w_p),  d lse / d L_p = w_p.
 * So, for the upstream gradients g (of out, D values) and g_lse (of lse_out):
 *   dO_p = w_p g,
 *   dL_p = w_p (<g, O_p> - <g, out> + g_lse)   for p in V,
 * and both are zero outside V (an invalid or masked partial does not enter
 * the combine).  An empty V gives zeros throughout.  The weights are formed as
 * in orc_combine_row_f64 (max subtracted first) and normalised by Z.
 */
void orc_combine_row_backward_f64(const double* part_o, const double* part_l, const int* valid,
                                  int64_t P, int64_t D, const double* g, double g_lse,
                                  double* d_o, double* d_l)
{
    double M = -INFINITY;
    int any = 0;
    for (int64_t p = 0; p < P; ++p) {
        d_l[p] = 0.0;
        for (int64_t d = 0; d < D; ++d)
            d_o[p * D + d] = 0.0;
        if (valid[p] && isfinite(part_l[p])) {
            if (!any || part_l[p] > M)
                M = part_l[p];
            any = 1;
        }
    }
    if (!any)
        return;
    double Z = 0.0;
    for (int64_t p = 0; p < P; ++p)
        if (valid[p] && isfinite(part_l[p]))
            Z += exp(part_l[p] - M);
    /* <g, out> with out = sum w_p O_p */
    double g_out = 0.0;
    for (int64_t d = 0; d < D; ++d) {
        double o = 0.0;
        for (int64_t p = 0; p < P; ++p)
            if (valid[p] && isfinite(part_l[p]))
                o += exp(part_l[p] - M) / Z * part_o[p * D + d];
        g_out += g[d] * o;
    }
    for (int64_t p = 0; p < P; ++p) {
        if (!(valid[p] && isfinite(part_l[p])))
            continue;
        double w = exp(part_l[p] - M) / Z;
        double gp = 0.0;
        for (int64_t d = 0; d < D; ++d) {
            gp += g[d] * part_o[p * D + d];
            d_o[p * D + d] = w * g[d];
        }
        d_l[p] = w * (gp - g_out + g_lse);
    }
}

/*
 * Typed strided gradient of orc_lse_combine over rows (t, h), t in
 * [t_begin, t_end), the pointers addressing row t_begin as there:
 *   g_out       (t, h, d) at go_st*(t - t_begin) + go_sh*h + d       (payload dtype)
 *   g_lse       (t, h)    at gl_st*(t - t_begin) + gl_sh*h (nullable: zero)
 *   d_part_out  (p, t, h, d) at dpo_sp*p + dpo_st*(t - t_begin) + dpo_sh*h + d
 *   d_part_lse  (p, t, h)    at dpl_sp*p + dpl_st*(t - t_begin) + dpl_sh*h  (fp32)
 * With cu_seqlens non-null the causal piece rule gates partial p as in the
 * forward.  dO is rounded once to the payload dtype, dL once to fp32; the O row
 * of a partial outside V is not read.
 */
void orc_lse_combine_backward(const void* part_out, int64_t po_sp, int64_t po_st, int64_t po_sh,
                              const float* part_lse, int64_t pl_sp, int64_t pl_st, int64_t pl_sh,
                              int64_t P, int64_t t_begin, int64_t t_end, int64_t H, int64_t D,
                              int dtype, const void* g_out, int64_t go_st, int64_t go_sh,
                              const float* g_lse, int64_t gl_st, int64_t gl_sh, void* d_part_out,
                              int64_t dpo_sp, int64_t dpo_st, int64_t dpo_sh, float* d_part_lse,
                              int64_t dpl_sp, int64_t dpl_st, int64_t dpl_sh,
                              const int32_t* cu_seqlens, int64_t nseq)
{
    double* po = (double*)malloc(sizeof(double) * (size_t)(P * D + 1));
    double* pl = (double*)malloc(sizeof(double) * (size_t)(P + 1));
    int* valid = (int*)malloc(sizeof(int) * (size_t)(P + 1));
    double* g = (double*)malloc(sizeof(double) * (size_t)(D + 1));
    double* d_o = (double*)malloc(sizeof(double) * (size_t)(P * D + 1));
    double* d_l = (double*)malloc(sizeof(double) * (size_t)(P + 1));
    for (int64_t t = t_begin; t < t_end; ++t)
        for (int64_t h = 0; h < H; ++h) {
            int64_t tr = t - t_begin;
            for (int64_t p = 0; p < P; ++p) {
                valid[p] = cu_seqlens ? orc_causal_piece_valid(cu_seqlens, nseq, P, p, t) : 1;
                pl[p] = -INFINITY;
                if (!valid[p])
                    continue;
                pl[p] = (double)part_lse[p * pl_sp + tr * pl_st + h * pl_sh];
                if (!isfinite(pl[p]))
                    continue;
                for (int64_t d = 0; d < D; ++d)
                    po[p * D + d] = load_half(part_out, p * po_sp + tr * po_st + h * po_sh + d, dtype);
            }
            for (int64_t d = 0; d < D; ++d)
                g[d] = load_half(g_out, tr * go_st + h * go_sh + d, dtype);
            double gl = g_lse ? (double)g_lse[tr * gl_st + h * gl_sh] : 0.0;
            orc_combine_row_backward_f64(po, pl, valid, P, D, g, gl, d_o, d_l);
            for (int64_t p = 0; p < P; ++p) {
                for (int64_t d = 0; d < D; ++d)
                    store_half(d_part_out, p * dpo_sp + tr * dpo_st + h * dpo_sh + d, dtype, d_o[p * D + d]);
                d_part_lse[p * dpl_sp + tr * dpl_st + h * dpl_sh] = (float)d_l[p];
            }
        }
    free(po);
    free(pl);
    free(valid);
    free(g);
    free(d_o);
    free(d_l);
}

/* ------------------------------------------------------------------------ */
/* THD layout planner and planned-span relayout  ([CU] PR description)        */
/* ------------------------------------------------------------------------ */
/*
 * The page states what the planner must achieve, not its steps: even
 * per-rank work, counting both the part proportional to tokens and the
 * causal part that grows with position, for any packed THD batch over the
 * context-parallel ranks; shards made of aligned blocks, every rank holding
 * the same number of blocks up to one (any rank count, not only powers of
 * two); a short sample left on one rank; long sequences dealt out in a
 * direction that flips from rank to rank; several grids tried, each a
 * greedy assignment followed by moving tokens between ranks, with the plain
 * contiguous layout kept as a candidate; the same spans for the same input;
 * and its input rules (positive block size, block-aligned min_split_tokens and lengths,
 * positive max_chunks_per_rank, finite non-negative weights not both zero,
 * at least one block per rank).  Reading (the concrete algorithm):
 *
 *  n_i = L_i / b blocks, N = sum n_i; rank r holds exactly
 *  cap_r = floor((r+1)N/W) - floor(rN/W) blocks (the balanced shards).
 *  Work of a token at position k of its sequence: token_weight
 *  + causal_weight * (k + 1) (a causal query sees k + 1 keys); a rank's cost
 *  is token_weight * tokens + causal_weight * sum(k + 1) over its tokens.
 *  Candidate 0 (contiguous): rank r takes global blocks
 *  [floor(rN/W), floor((r+1)N/W)).  Candidate g = 1..6 (grid g): a sequence
 *  is long if L_i >= min_split_tokens (and n_i >= 2), else short.
 *   B. shorts, costliest first (ties: batch order), each whole to the
 *      cheapest rank (ties: lowest) with room for it; a short that fits
 *      nowhere waits for C2 (placing the shorts first splits a short only
 *      when it does not fit beside the shorts already placed);
 *   A. then each long sequence (the l-th, in batch order) is cut into
 *      m = min(n_i, W * 2^(g-1)) chunks [floor(c n_i/m), floor((c+1) n_i/m));
 *      chunk c goes to rank psi = c mod W if floor(c/W) + l is even, else to
 *      W - 1 - psi (a snake whose direction alternates per round and per
 *      long sequence), capacity notwithstanding;
 *   C1. while a rank is over capacity (only long chunks overfill): the
 *      lowest such rank o moves x = min(excess of o, room of u, span length)
 *      blocks to the cheapest rank u with room (ties: lowest): either the
 *      last blocks of its long-sequence span ending highest (ties: later
 *      sequence) or the first blocks of its long-sequence span starting
 *      lowest (ties: earlier sequence), whichever leaves the larger of the
 *      two ranks' costs smaller (ties: the last blocks);
 *   C2. each waiting short, in B's order, is laid into the cheapest ranks
 *      with room, in order, as far as their room allows;
 *   D. up to 4W exchanges between the costliest and the cheapest rank (ties:
 *      lowest): the costliest gives the last x blocks of its long-sequence
 *      span ending highest, the cheapest gives the first x blocks of its
 *      long-sequence span starting lowest (token counts stay exact), x chosen
 *      to minimise the larger of the two costs (ties: smallest x); stop when
 *      no exchange lowers it;
 *   then spans of one sequence that meet on one rank are merged, and a
 *   candidate with more than max_chunks_per_rank spans on a rank is dropped.
 *  The plan is the candidate with the least maximum rank cost, ties to fewer
 *  spans, then to the lower candidate number (so the contiguous layout wins
 *  ties and is the fallback).
 *
 *  Output: spans in packed token order: span_start[n + 1] (global token of
 *  each span's first row, span_start[n] = T), span_rank[n], span_local[n]
 *  (the span's first row within its rank's slab; a rank's slab lists its
 *  spans in packed order), rank_off[W + 1] (token prefix of the slabs),
 *  rank_cost[W], and the chosen candidate.  Returns 0, or a negative code:
 *  -1 bad config or world size, -2 misaligned or malformed lengths,
 *  -3 fewer blocks than ranks, -4 span capacity too small (*n_spans is then
 *  the count needed).
 */
typedef struct {
    int64_t seq, a, e, rank; /* blocks [a, e) of sequence seq */
} orc_span;

typedef struct {
    orc_span* s;
    int64_t n, cap;
} orc_spans;

/* Optional record of the rebalancing steps C1 and C2 (test instrumentation;
 * it changes no decision): per C1 move and per C2 piece, the ranks, the
 * candidate spans, the blocks moved or placed, and every rank's blocks and
 * causal work just before. */
#define ORC_TRACE_MAX_W 16
typedef struct {
    int64_t step;                   /* 1: C1 move, 2: C2 piece */
    int64_t over, to;               /* C1: overfull and receiving rank; C2: -1 and receiving rank */
    int64_t amount;                 /* C1: min(excess of over, room of to); C2: blocks placed */
    int64_t top_seq, top_a, top_e;  /* C1: o's long span ending highest, before the move */
    int64_t bot_seq, bot_a, bot_e;  /* C1: o's long span starting lowest, before the move */
    int64_t chose_bottom;           /* C1 */
    int64_t moved_seq, moved_a, moved_e;
    int64_t blk[ORC_TRACE_MAX_W], caus[ORC_TRACE_MAX_W];
} orc_plan_trace;

typedef struct {
    orc_plan_trace* rec;
    int64_t cap, n;
} orc_trace_buf;

static void spans_add(orc_spans* v, int64_t seq, int64_t a, int64_t e, int64_t rank)
{
    if (a >= e)
        return;
    if (v->n == v->cap) {
        v->cap = v->cap ? 2 * v->cap : 64;
        v->s = (orc_span*)realloc(v->s, sizeof(orc_span) * (size_t)v->cap);
    }
    v->s[v->n].seq = seq;
    v->s[v->n].a = a;
    v->s[v->n].e = e;
    v->s[v->n].rank = rank;
    v->n++;
}

/* 1 + 2 + ... + n */
static int64_t tri(int64_t n) { return n * (n + 1) / 2; }

/* sum of (k + 1) over token positions k in [ta, te) */
static int64_t causal_work(int64_t ta, int64_t te) { return tri(te) - tri(ta); }

static double work_cost(double wt, double wc, int64_t tokens, int64_t causal)
{
    double x = wt * (double)tokens;
    double y = wc * (double)causal;
    return x + y;
}

typedef struct {
    int64_t W, b;
    double wt, wc;
    int64_t *blk, *caus; /* per rank: blocks and causal work held */
    const int64_t* capb;
} orc_loads;

static double rank_cost_of(const orc_loads* L, int64_t r)
{
    return work_cost(L->wt, L->wc, L->blk[r] * L->b, L->caus[r]);
}

static void loads_add(orc_loads* L, int64_t r, int64_t a, int64_t e, int sign)
{
    L->blk[r] += sign * (e - a);
    L->caus[r] += sign * causal_work(a * L->b, e * L->b);
}

/* cheapest rank with room for `need` blocks (ties: lowest), -1 if none */
static int64_t cheapest_with_room(const orc_loads* L, int64_t need)
{
    int64_t best = -1;
    for (int64_t r = 0; r < L->W; ++r)
        if (L->capb[r] - L->blk[r] >= need && (best < 0 || rank_cost_of(L, r) < rank_cost_of(L, best)))
            best = r;
    return best;
}

static int span_order(const void* x, const void* y)
{
    const orc_span* p = (const orc_span*)x;
    const orc_span* q = (const orc_span*)y;
    if (p->seq != q->seq)
        return p->seq < q->seq ? -1 : 1;
    return p->a < q->a ? -1 : (p->a > q->a ? 1 : 0);
}

/* merge spans of one sequence that meet on one rank (spans sorted) */
static void spans_normalize(orc_spans* v)
{
    qsort(v->s, (size_t)v->n, sizeof(orc_span), span_order);
    int64_t m = 0;
    for (int64_t k = 0; k < v->n; ++k) {
        if (m > 0 && v->s[m - 1].seq == v->s[k].seq && v->s[m - 1].rank == v->s[k].rank && v->s[m - 1].e == v->s[k].a)
            v->s[m - 1].e = v->s[k].e;
        else
            v->s[m++] = v->s[k];
    }
    v->n = m;
}

/* grid g >= 1, or the contiguous layout for g = 0 */
static orc_plan_trace* trace_next(orc_trace_buf* tb, const orc_loads* L)
{
    if (!tb || L->W > ORC_TRACE_MAX_W)
        return NULL;
    orc_plan_trace* t = tb->n < tb->cap ? &tb->rec[tb->n] : NULL;
    tb->n++;
    if (t) {
        memset(t, 0, sizeof(*t));
        for (int64_t r = 0; r < L->W; ++r) {
            t->blk[r] = L->blk[r];
            t->caus[r] = L->caus[r];
        }
    }
    return t;
}

static void plan_candidate(int g, const int64_t* nb, int64_t nseq, int64_t W, int64_t b, int64_t min_split,
                           double wt, double wc, const int64_t* capb, orc_spans* out, orc_trace_buf* tb)
{
    int64_t* blk = (int64_t*)calloc((size_t)W, sizeof(int64_t));
    int64_t* caus = (int64_t*)calloc((size_t)W, sizeof(int64_t));
    orc_loads L = {W, b, wt, wc, blk, caus, capb};
    out->n = 0;
    if (g == 0) {
        int64_t N = 0;
        for (int64_t i = 0; i < nseq; ++i)
            N += nb[i];
        int64_t base = 0;
        for (int64_t i = 0; i < nseq; ++i) {
            for (int64_t r = 0; r < W; ++r) {
                int64_t lo = r * N / W, hi = (r + 1) * N / W;
                int64_t a = lo > base ? lo - base : 0;
                int64_t e = hi - base < nb[i] ? hi - base : nb[i];
                spans_add(out, i, a, e, r);
            }
            base += nb[i];
        }
    } else {
        const int64_t M = W << (g - 1);
        /* B: shorts, costliest first, whole where they fit (before any long chunk) */
        int64_t* order = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nseq + 1));
        int64_t ns = 0;
        for (int64_t i = 0; i < nseq; ++i)
            if (nb[i] > 0 && !(nb[i] * b >= min_split && nb[i] >= 2))
                order[ns++] = i;
        for (int64_t x = 1; x < ns; ++x) /* insertion sort: cost desc, index asc */
            for (int64_t y = x; y > 0; --y) {
                int64_t i = order[y - 1], j = order[y];
                double ci = work_cost(wt, wc, nb[i] * b, causal_work(0, nb[i] * b));
                double cj = work_cost(wt, wc, nb[j] * b, causal_work(0, nb[j] * b));
                if (cj > ci || (cj == ci && j < i)) {
                    order[y - 1] = j;
                    order[y] = i;
                } else {
                    break;
                }
            }
        int64_t* aside = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nseq + 1));
        int64_t na = 0;
        for (int64_t x = 0; x < ns; ++x) {
            int64_t i = order[x];
            int64_t r = cheapest_with_room(&L, nb[i]);
            if (r < 0) {
                aside[na++] = i;
                continue;
            }
            spans_add(out, i, 0, nb[i], r);
            loads_add(&L, r, 0, nb[i], +1);
        }
        /* A: long sequences, snake */
        int64_t ell = 0;
        for (int64_t i = 0; i < nseq; ++i) {
            if (!(nb[i] * b >= min_split && nb[i] >= 2))
                continue;
            int64_t m = nb[i] < M ? nb[i] : M;
            for (int64_t c = 0; c < m; ++c) {
                int64_t a = c * nb[i] / m, e = (c + 1) * nb[i] / m;
                int64_t psi = c % W;
                int64_t r = ((c / W + ell) % 2 == 0) ? psi : W - 1 - psi;
                spans_add(out, i, a, e, r);
                loads_add(&L, r, a, e, +1);
            }
            ell++;
        }
        /* C1: rebalance to exact capacity */
        for (;;) {
            int64_t o = -1;
            for (int64_t r = 0; r < W && o < 0; ++r)
                if (blk[r] > capb[r])
                    o = r;
            if (o < 0)
                break;
            /* two candidate moves: the last blocks of o's long span that ends
             * highest (ties: later sequence), or the first blocks of its long
             * span that starts lowest (ties: earlier sequence) */
            int64_t dh = -1, dl = -1;
            for (int64_t k = 0; k < out->n; ++k) {
                const orc_span* s = &out->s[k];
                if (s->rank != o || s->a >= s->e || !(nb[s->seq] * b >= min_split && nb[s->seq] >= 2))
                    continue;
                if (dh < 0 || s->e > out->s[dh].e || (s->e == out->s[dh].e && s->seq > out->s[dh].seq))
                    dh = k;
                if (dl < 0 || s->a < out->s[dl].a || (s->a == out->s[dl].a && s->seq < out->s[dl].seq))
                    dl = k;
            }
            int64_t u = cheapest_with_room(&L, 1);
            int64_t x = blk[o] - capb[o];
            if (capb[u] - blk[u] < x)
                x = capb[u] - blk[u];
            int64_t xh = out->s[dh].e - out->s[dh].a < x ? out->s[dh].e - out->s[dh].a : x;
            int64_t xl = out->s[dl].e - out->s[dl].a < x ? out->s[dl].e - out->s[dl].a : x;
            /* the larger of o's and u's costs after each move */
            int64_t eh = out->s[dh].e, al = out->s[dl].a;
            loads_add(&L, o, eh - xh, eh, -1);
            loads_add(&L, u, eh - xh, eh, +1);
            double co = rank_cost_of(&L, o), cu = rank_cost_of(&L, u);
            double mh = co > cu ? co : cu;
            loads_add(&L, u, eh - xh, eh, -1);
            loads_add(&L, o, eh - xh, eh, +1);
            loads_add(&L, o, al, al + xl, -1);
            loads_add(&L, u, al, al + xl, +1);
            co = rank_cost_of(&L, o);
            cu = rank_cost_of(&L, u);
            double ml = co > cu ? co : cu;
            loads_add(&L, u, al, al + xl, -1);
            loads_add(&L, o, al, al + xl, +1);
            orc_plan_trace* tr = trace_next(tb, &L);
            if (tr) {
                tr->step = 1;
                tr->over = o;
                tr->to = u;
                tr->amount = x;
                tr->top_seq = out->s[dh].seq;
                tr->top_a = out->s[dh].a;
                tr->top_e = out->s[dh].e;
                tr->bot_seq = out->s[dl].seq;
                tr->bot_a = out->s[dl].a;
                tr->bot_e = out->s[dl].e;
                tr->chose_bottom = ml < mh;
                tr->moved_seq = ml < mh ? out->s[dl].seq : out->s[dh].seq;
                tr->moved_a = ml < mh ? al : eh - xh;
                tr->moved_e = ml < mh ? al + xl : eh;
            }
            if (ml < mh) {
                int64_t seq = out->s[dl].seq;
                out->s[dl].a = al + xl;
                loads_add(&L, o, al, al + xl, -1);
                spans_add(out, seq, al, al + xl, u);
                loads_add(&L, u, al, al + xl, +1);
            } else {
                int64_t seq = out->s[dh].seq;
                out->s[dh].e = eh - xh;
                loads_add(&L, o, eh - xh, eh, -1);
                spans_add(out, seq, eh - xh, eh, u);
                loads_add(&L, u, eh - xh, eh, +1);
            }
        }
        /* C2: shorts that fit nowhere whole */
        for (int64_t x = 0; x < na; ++x) {
            int64_t i = aside[x];
            int64_t a = 0;
            while (a < nb[i]) {
                int64_t u = cheapest_with_room(&L, 1);
                int64_t k = capb[u] - blk[u];
                if (nb[i] - a < k)
                    k = nb[i] - a;
                orc_plan_trace* tr = trace_next(tb, &L);
                if (tr) {
                    tr->step = 2;
                    tr->over = -1;
                    tr->to = u;
                    tr->amount = k;
                    tr->moved_seq = i;
                    tr->moved_a = a;
                    tr->moved_e = a + k;
                }
                spans_add(out, i, a, a + k, u);
                loads_add(&L, u, a, a + k, +1);
                a += k;
            }
        }
        /* D: exchanges between the costliest and the cheapest rank (ties:
         * lowest rank), at most 4W: the costliest gives the last x blocks of
         * its long span ending highest, the cheapest the first x blocks of its
         * long span starting lowest (token counts unchanged); x minimises the
         * larger of their two costs; stop when no exchange lowers it */
        for (int64_t round = 0; round < 4 * W; ++round) {
            int64_t hi = 0, lo = 0;
            for (int64_t r = 1; r < W; ++r) {
                if (rank_cost_of(&L, r) > rank_cost_of(&L, hi))
                    hi = r;
                if (rank_cost_of(&L, r) < rank_cost_of(&L, lo))
                    lo = r;
            }
            if (hi == lo)
                break;
            int64_t dh = -1, dl = -1;
            for (int64_t k = 0; k < out->n; ++k) {
                const orc_span* s = &out->s[k];
                if (s->a >= s->e || !(nb[s->seq] * b >= min_split && nb[s->seq] >= 2))
                    continue;
                if (s->rank == hi &&
                    (dh < 0 || s->e > out->s[dh].e || (s->e == out->s[dh].e && s->seq > out->s[dh].seq)))
                    dh = k;
                if (s->rank == lo &&
                    (dl < 0 || s->a < out->s[dl].a || (s->a == out->s[dl].a && s->seq < out->s[dl].seq)))
                    dl = k;
            }
            if (dh < 0 || dl < 0)
                break;
            const double c_hi = rank_cost_of(&L, hi), c_lo = rank_cost_of(&L, lo);
            double now = c_hi > c_lo ? c_hi : c_lo;
            int64_t eh = out->s[dh].e, al = out->s[dl].a;
            int64_t xmax = out->s[dh].e - out->s[dh].a;
            if (out->s[dl].e - out->s[dl].a < xmax)
                xmax = out->s[dl].e - out->s[dl].a;
            int64_t best_x = 0;
            double best = now;
            for (int64_t x = 1; x <= xmax; ++x) {
                loads_add(&L, hi, eh - x, eh, -1);
                loads_add(&L, lo, eh - x, eh, +1);
                loads_add(&L, lo, al, al + x, -1);
                loads_add(&L, hi, al, al + x, +1);
                double a1 = rank_cost_of(&L, hi), a2 = rank_cost_of(&L, lo);
                double m = a1 > a2 ? a1 : a2;
                loads_add(&L, hi, al, al + x, -1);
                loads_add(&L, lo, al, al + x, +1);
                loads_add(&L, lo, eh - x, eh, -1);
                loads_add(&L, hi, eh - x, eh, +1);
                if (m < best) {
                    best = m;
                    best_x = x;
                }
            }
            if (best_x == 0)
                break;
            int64_t sh = out->s[dh].seq, sl = out->s[dl].seq;
            out->s[dh].e = eh - best_x;
            out->s[dl].a = al + best_x;
            loads_add(&L, hi, eh - best_x, eh, -1);
            loads_add(&L, lo, al, al + best_x, -1);
            spans_add(out, sh, eh - best_x, eh, lo);
            loads_add(&L, lo, eh - best_x, eh, +1);
            spans_add(out, sl, al, al + best_x, hi);
            loads_add(&L, hi, al, al + best_x, +1);
        }
        free(order);
        free(aside);
        /* drop spans emptied by C1 and D */
        int64_t m = 0;
        for (int64_t k = 0; k < out->n; ++k)
            if (out->s[k].a < out->s[k].e)
                out->s[m++] = out->s[k];
        out->n = m;
    }
    spans_normalize(out);
    free(blk);
    free(caus);
}

int orc_thd_plan(const int32_t* cu, int64_t nseq, int64_t W, int64_t block_size, int64_t min_split_tokens,
                 int64_t max_chunks_per_rank, double token_weight, double causal_weight, int64_t max_spans,
                 int32_t* span_start, int32_t* span_rank, int32_t* span_local, int64_t* rank_off,
                 double* rank_cost, int64_t* n_spans, int32_t* chosen)
{
    const int64_t b = block_size;
    if (W < 1 || b < 1 || min_split_tokens < 1 || min_split_tokens % b != 0 || max_chunks_per_rank < 1 ||
        !isfinite(token_weight) || !isfinite(causal_weight) || token_weight < 0 || causal_weight < 0 ||
        (token_weight == 0 && causal_weight == 0))
        return -1;
    if (nseq < 0 || cu[0] != 0)
        return -2;
    int64_t* nb = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nseq + 1));
    int64_t N = 0;
    for (int64_t i = 0; i < nseq; ++i) {
        int64_t L = (int64_t)cu[i + 1] - cu[i];
        if (L < 0 || L % b != 0) {
            free(nb);
            return -2;
        }
        nb[i] = L / b;
        N += nb[i];
    }
    if (N < W) {
        free(nb);
        return -3;
    }
    int64_t* capb = (int64_t*)malloc(sizeof(int64_t) * (size_t)W);
    for (int64_t r = 0; r < W; ++r)
        capb[r] = (r + 1) * N / W - r * N / W;

    orc_spans best = {0, 0, 0}, cand = {0, 0, 0};
    double best_max = 0.0;
    int best_g = -1;
    int64_t* blk = (int64_t*)malloc(sizeof(int64_t) * (size_t)W);
    int64_t* caus = (int64_t*)malloc(sizeof(int64_t) * (size_t)W);
    int64_t* cnt = (int64_t*)malloc(sizeof(int64_t) * (size_t)W);
    for (int g = 0; g <= 6; ++g) {
        plan_candidate(g, nb, nseq, W, b, min_split_tokens, token_weight, causal_weight, capb, &cand, NULL);
        for (int64_t r = 0; r < W; ++r)
            blk[r] = caus[r] = cnt[r] = 0;
        for (int64_t k = 0; k < cand.n; ++k) {
            const orc_span* s = &cand.s[k];
            blk[s->rank] += s->e - s->a;
            caus[s->rank] += causal_work(s->a * b, s->e * b);
            cnt[s->rank]++;
        }
        int fits = 1;
        double mx = 0.0;
        for (int64_t r = 0; r < W; ++r) {
            if (cnt[r] > max_chunks_per_rank)
                fits = 0;
            double c = work_cost(token_weight, causal_weight, blk[r] * b, caus[r]);
            if (r == 0 || c > mx)
                mx = c;
        }
        if (g > 0 && !fits)
            continue;
        if (best_g < 0 || mx < best_max || (mx == best_max && cand.n < best.n)) {
            orc_spans t = best;
            best = cand;
            cand = t;
            best_max = mx;
            best_g = g;
        }
    }
    free(cand.s);
    *n_spans = best.n;
    int rc = 0;
    if (best.n > max_spans) {
        rc = -4;
    } else {
        int64_t* fill = (int64_t*)calloc((size_t)W, sizeof(int64_t));
        rank_off[0] = 0;
        for (int64_t r = 0; r < W; ++r) {
            rank_off[r + 1] = rank_off[r] + capb[r] * b;
            blk[r] = caus[r] = 0;
        }
        for (int64_t k = 0; k < best.n; ++k) {
            const orc_span* s = &best.s[k];
            span_start[k] = (int32_t)(cu[s->seq] + s->a * b);
            span_rank[k] = (int32_t)s->rank;
            span_local[k] = (int32_t)fill[s->rank];
            fill[s->rank] += (s->e - s->a) * b;
            blk[s->rank] += s->e - s->a;
            caus[s->rank] += causal_work(s->a * b, s->e * b);
        }
        span_start[best.n] = cu[nseq];
        for (int64_t r = 0; r < W; ++r)
            rank_cost[r] = work_cost(token_weight, causal_weight, blk[r] * b, caus[r]);
        *chosen = best_g;
        free(fill);
    }
    free(best.s);
    free(nb);
    free(capb);
    free(blk);
    free(caus);
    free(cnt);
    return rc;
}

/*
 * One candidate of orc_thd_plan (g = 0 contiguous, g >= 1 a grid) with the
 * record of its rebalancing steps C1 and C2 (test instrumentation: the tests
 * recompute each decision from the recorded loads).  Writes up to max_trace
 * records and sets *n_trace to the number made (W <= 16 for records), and
 * the candidate's spans (sequence, first block, end block, rank) up to
 * max_spans, *n_spans to their number.  Returns 0, or -1 .. -3 as
 * orc_thd_plan.
 */
int orc_thd_plan_candidate_trace(const int32_t* cu, int64_t nseq, int64_t W, int64_t block_size,
                                 int64_t min_split_tokens, double token_weight, double causal_weight, int g,
                                 orc_plan_trace* trace, int64_t max_trace, int64_t* n_trace, int64_t* spans,
                                 int64_t max_spans, int64_t* n_spans)
{
    const int64_t b = block_size;
    if (W < 1 || b < 1 || min_split_tokens < 1 || min_split_tokens % b != 0 || g < 0 || g > 6)
        return -1;
    if (nseq < 0 || cu[0] != 0)
        return -2;
    int64_t* nb = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nseq + 1));
    int64_t N = 0;
    for (int64_t i = 0; i < nseq; ++i) {
        int64_t L = (int64_t)cu[i + 1] - cu[i];
        if (L < 0 || L % b != 0) {
            free(nb);
            return -2;
        }
        nb[i] = L / b;
        N += nb[i];
    }
    if (N < W) {
        free(nb);
        return -3;
    }
    int64_t* capb = (int64_t*)malloc(sizeof(int64_t) * (size_t)W);
    for (int64_t r = 0; r < W; ++r)
        capb[r] = (r + 1) * N / W - r * N / W;
    orc_spans cand = {0, 0, 0};
    orc_trace_buf tb = {trace, max_trace, 0};
    plan_candidate(g, nb, nseq, W, b, min_split_tokens, token_weight, causal_weight, capb, &cand, &tb);
    *n_trace = tb.n;
    *n_spans = cand.n;
    for (int64_t k = 0; k < cand.n && k < max_spans; ++k) {
        spans[4 * k + 0] = cand.s[k].seq;
        spans[4 * k + 1] = cand.s[k].a;
        spans[4 * k + 2] = cand.s[k].e;
        spans[4 * k + 3] = cand.s[k].rank;
    }
    free(cand.s);
    free(nb);
    free(capb);
    return 0;
}

/*
 * Relayout over planned spans (B planes, D contiguous, es-byte elements):
 *   sequence side: rank p's slab [B][T_p][H][D] at token row B*rank_off[p];
 *   head side:     [P][B][T][H/P][D] in packed token order.
 * Token t of span s (span_start[s] <= t < span_start[s+1]) is row
 * span_local[s] + t - span_start[s] of rank span_rank[s]'s slab.  dir 1:
 * sequence side -> head side; dir 0: the inverse.
 */
static void span_relayout(const void* in, void* out, const int32_t* span_start, const int32_t* span_rank,
                          const int32_t* span_local, const int64_t* rank_off, int64_t n_spans, int64_t P,
                          int64_t B, int64_t H, int64_t D, int64_t es, int dir)
{
    const int64_t T = span_start[n_spans];
    const int64_t Hp = H / P;
    const int64_t run = Hp * D * es;
    for (int64_t s = 0; s < n_spans; ++s) {
        const int64_t p = span_rank[s];
        const int64_t Tp = rank_off[p + 1] - rank_off[p];
        for (int64_t t = span_start[s]; t < span_start[s + 1]; ++t) {
            const int64_t l = span_local[s] + (t - span_start[s]);
            for (int64_t bb = 0; bb < B; ++bb) {
                const int64_t seq_row = B * rank_off[p] + bb * Tp + l;
                for (int64_t r = 0; r < P; ++r) {
                    const int64_t head_row = (r * B + bb) * T + t;
                    char* sq = (char*)(dir ? in : out) + (seq_row * H + r * Hp) * D * es;
                    char* hd = (char*)(dir ? out : in) + head_row * Hp * D * es;
                    if (dir)
                        memcpy(hd, sq, (size_t)run);
                    else
                        memcpy(sq, hd, (size_t)run);
                }
            }
        }
    }
}

void orc_span_seq_to_head(const void* in, void* out, const int32_t* span_start, const int32_t* span_rank,
                          const int32_t* span_local, const int64_t* rank_off, int64_t n_spans, int64_t P,
                          int64_t B, int64_t H, int64_t D, int64_t es)
{
    span_relayout(in, out, span_start, span_rank, span_local, rank_off, n_spans, P, B, H, D, es, 1);
}

void orc_span_head_to_seq(const void* in, void* out, const int32_t* span_start, const int32_t* span_rank,
                          const int32_t* span_local, const int64_t* rank_off, int64_t n_spans, int64_t P,
                          int64_t B, int64_t H, int64_t D, int64_t es)
{
    span_relayout(in, out, span_start, span_rank, span_local, rank_off, n_spans, P, B, H, D, es, 0);
}

/* ------------------------------------------------------------------------ */
/* Causal combine over a THD layout plan                                      */
/* ------------------------------------------------------------------------ */
/*
 * Reading (context parallelism over a planned layout, [CU]): every rank holds
 * the queries and the keys of its spans; partial p of token (i, k) is the
 * causal attention of that query over the keys rank p holds of sequence i,
 * so it sees a key, and is valid, iff rank p holds a position <= k of
 * sequence i.  first_pos[p * nseq + i] is the smallest position of sequence i
 * that rank p holds (INT32_MAX if none).  For the per-sequence split this is
 * the piece rule of orc_causal_piece_valid.
 */
void orc_plan_first_positions(const int32_t* cu, int64_t nseq, int64_t W, const int32_t* span_start,
                              const int32_t* span_rank, int64_t n_spans, int32_t* first_pos)
{
    for (int64_t k = 0; k < W * nseq; ++k)
        first_pos[k] = INT32_MAX;
    for (int64_t s = 0; s < n_spans; ++s) {
        /* the sequence that contains the span's first token (a span is
         * non-empty and lies inside one sequence) */
        int64_t i = 0;
        while (!(span_start[s] >= cu[i] && span_start[s] < cu[i + 1]))
            ++i;
        int64_t pos = (int64_t)span_start[s] - cu[i];
        int32_t* f = &first_pos[(int64_t)span_rank[s] * nseq + i];
        if (pos < *f)
            *f = (int32_t)pos;
    }
}

int orc_plan_piece_valid(const int32_t* cu, int64_t nseq, const int32_t* first_pos, int64_t p, int64_t t)
{
    for (int64_t i = 0; i < nseq; ++i)
        if (t >= cu[i] && t < cu[i + 1])
            return (int64_t)first_pos[p * nseq + i] <= t - cu[i];
    return 0;
}

/* orc_lse_combine with the planned validity rule (layouts as there). */
void orc_lse_combine_planned(const void* part_out, int64_t po_sp, int64_t po_st, int64_t po_sh,
                             const float* part_lse, int64_t pl_sp, int64_t pl_st, int64_t pl_sh, int64_t P,
                             int64_t t_begin, int64_t t_end, int64_t H, int64_t D, int dtype, void* out,
                             int64_t o_st, int64_t o_sh, float* lse_out, int64_t lo_st, int64_t lo_sh,
                             const int32_t* cu_seqlens, const int32_t* first_pos, int64_t nseq)
{
    double* po = (double*)malloc(sizeof(double) * (size_t)(P * D + 1));
    double* pl = (double*)malloc(sizeof(double) * (size_t)(P + 1));
    int* valid = (int*)malloc(sizeof(int) * (size_t)(P + 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)(D + 1));
    for (int64_t t = t_begin; t < t_end; ++t)
        for (int64_t h = 0; h < H; ++h) {
            int64_t tr = t - t_begin;
            for (int64_t p = 0; p < P; ++p) {
                valid[p] = orc_plan_piece_valid(cu_seqlens, nseq, first_pos, p, t);
                pl[p] = -INFINITY;
                if (!valid[p])
                    continue;
                pl[p] = (double)part_lse[p * pl_sp + tr * pl_st + h * pl_sh];
                if (!isfinite(pl[p]))
                    continue;
                for (int64_t d = 0; d < D; ++d)
                    po[p * D + d] = load_half(part_out, p * po_sp + tr * po_st + h * po_sh + d, dtype);
            }
            double lse;
            orc_combine_row_f64(po, pl, valid, P, D, acc, &lse);
            for (int64_t d = 0; d < D; ++d)
                store_half(out, tr * o_st + h * o_sh + d, dtype, acc[d]);
            if (lse_out)
                lse_out[tr * lo_st + h * lo_sh] = (float)lse;
        }
    free(po);
    free(pl);
    free(valid);
    free(acc);
}

/* orc_lse_combine_backward with the planned validity rule. */
void orc_lse_combine_planned_backward(const void* part_out, int64_t po_sp, int64_t po_st, int64_t po_sh,
                                      const float* part_lse, int64_t pl_sp, int64_t pl_st, int64_t pl_sh,
                                      int64_t P, int64_t t_begin, int64_t t_end, int64_t H, int64_t D,
                                      int dtype, const void* g_out, int64_t go_st, int64_t go_sh,
                                      const float* g_lse, int64_t gl_st, int64_t gl_sh, void* d_part_out,
                                      int64_t dpo_sp, int64_t dpo_st, int64_t dpo_sh, float* d_part_lse,
                                      int64_t dpl_sp, int64_t dpl_st, int64_t dpl_sh,
                                      const int32_t* cu_seqlens, const int32_t* first_pos, int64_t nseq)
{
    double* po = (double*)malloc(sizeof(double) * (size_t)(P * D + 1));
    double* pl = (double*)malloc(sizeof(double) * (size_t)(P + 1));
    int* valid = (int*)malloc(sizeof(int) * (size_t)(P + 1));
    double* g = (double*)malloc(sizeof(double) * (size_t)(D + 1));
    double* d_o = (double*)malloc(sizeof(double) * (size_t)(P * D + 1));
    double* d_l = (double*)malloc(sizeof(double) * (size_t)(P + 1));
    for (int64_t t = t_begin; t < t_end; ++t)
        for (int64_t h = 0; h < H; ++h) {
            int64_t tr = t - t_begin;
            for (int64_t p = 0; p < P; ++p) {
                valid[p] = orc_plan_piece_valid(cu_seqlens, nseq, first_pos, p, t);
                pl[p] = -INFINITY;
                if (!valid[p])
                    continue;
                pl[p] = (double)part_lse[p * pl_sp + tr * pl_st + h * pl_sh];
                if (!isfinite(pl[p]))
                    continue;
                for (int64_t d = 0; d < D; ++d)
                    po[p * D + d] = load_half(part_out, p * po_sp + tr * po_st + h * po_sh + d, dtype);
            }
            for (int64_t d = 0; d < D; ++d)
                g[d] = load_half(g_out, tr * go_st + h * go_sh + d, dtype);
            double gl = g_lse ? (double)g_lse[tr * gl_st + h * gl_sh] : 0.0;
            orc_combine_row_backward_f64(po, pl, valid, P, D, g, gl, d_o, d_l);
            for (int64_t p = 0; p < P; ++p) {
                for (int64_t d = 0; d < D; ++d)
                    store_half(d_part_out, p * dpo_sp + tr * dpo_st + h * dpo_sh + d, dtype, d_o[p * D + d]);
                d_part_lse[p * dpl_sp + tr * dpl_st + h * dpl_sh] = (float)d_l[p];
            }
        }
    free(po);
    free(pl);
    free(valid);
    free(g);
    free(d_o);
    free(d_l);
}

/* ------------------------------------------------------------------------ */
/* Q/K/V projection into the head-sharded layout  ([FV] direct output slices) */
/* ------------------------------------------------------------------------ */
/*
 * out[r][b][t][h'][d] = sum_k x[t][k] * w[(b*H + r*H/P + h')*D + d][k]: the
 * projection of the stacked sequence shards x [S][K] by the fused weight
 * w [B*H*D][K] (a linear layer's layout), written where the seq->head
 * relayout of its result would put it.  Double accumulation, rounded once to
 * the payload type (dtype 0 bf16, 1 fp16).
 */
void orc_qkv_projection(const void* x, const void* w, void* out, int64_t S, int64_t K, int64_t P, int64_t B,
                        int64_t H, int64_t D, int dtype)
{
    const int64_t Hp = H / P;
    double* xr = (double*)malloc(sizeof(double) * (size_t)(K + 1));
    for (int64_t t = 0; t < S; ++t) {
        for (int64_t k = 0; k < K; ++k)
            xr[k] = load_half(x, t * K + k, dtype);
        for (int64_t b = 0; b < B; ++b)
            for (int64_t h = 0; h < H; ++h)
                for (int64_t d = 0; d < D; ++d) {
                    const int64_t n = (b * H + h) * D + d;
                    double acc = 0.0;
                    for (int64_t k = 0; k < K; ++k)
                        acc += xr[k] * load_half(w, n * K + k, dtype);
                    const int64_t r = h / Hp, hp = h % Hp;
                    store_half(out, (((r * B + b) * S + t) * Hp + hp) * D + d, dtype, acc);
                }
    }
    free(xr);
}
