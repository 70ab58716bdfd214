// cam_api.cpp -- the extern "C" entry points declared in include/cam.h.
//
// Host-only: every argument is checked here before anything reaches the GPU
// (this file makes no HIP call), then a launch record is built and handed to
// one kernel launcher.  A rejected call launches nothing and writes nothing:
// FastVideo's fused all-to-all helper either declines before it starts or
// runs to the end (commit message of "[perf] Probe H3 chunked all-to-all
// with direct output slices"); the same rule, applied per call.
#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <utility>

#include "cam_internal.h"

namespace cam {

static thread_local char g_err[512];
static thread_local uint64_t g_launch[3];  // workgroups, threads, LDS bytes

cam_status set_error(cam_status s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

void clear_error() { g_err[0] = '\0'; }

void note_launch(uint64_t workgroups, uint32_t threads, uint64_t lds_bytes)
{
    g_launch[0] = workgroups;
    g_launch[1] = threads;
    g_launch[2] = lds_bytes;
}

namespace {

constexpr int64_t kI64Max = INT64_MAX;
// Element strides beyond 2^48 address no real buffer; bounding them keeps every
// byte-stride and offset product of the launch records inside 64 bits.
constexpr int64_t kMaxStride = int64_t(1) << 48;

bool mul_ok(int64_t a, int64_t b, int64_t* out)
{
    if (a < 0 || b < 0)
        return false;
    if (a != 0 && b > kI64Max / a)
        return false;
    *out = a * b;
    return true;
}

bool prod_ok(std::initializer_list<int64_t> xs, int64_t* out)
{
    int64_t acc = 1;
    for (int64_t x : xs)
        if (!mul_ok(acc, x, &acc))
            return false;
    *out = acc;
    return true;
}

int elem_size(cam_dtype dt)
{
    switch (dt) {
    case CAM_BF16:
    case CAM_FP16:
        return 2;
    case CAM_FP32:
        return 4;
    default:  // any other code the enum's range admits
        return 0;
    }
}

const char* dt_name(cam_dtype dt)
{
    switch (dt) {
    case CAM_BF16: return "bf16";
    case CAM_FP16: return "fp16";
    case CAM_FP32: return "fp32";
    default: return "unknown";
    }
}

bool aligned(const void* p, int64_t n) { return (reinterpret_cast<uintptr_t>(p) % uint64_t(n)) == 0; }

// Widest access (16, 8, 4 or 2 bytes) that divides every byte quantity given.
int pick_width(std::initializer_list<uint64_t> quantities)
{
    for (int w : {16, 8, 4, 2}) {
        bool ok = true;
        for (uint64_t q : quantities)
            ok = ok && (q % uint64_t(w) == 0);
        if (ok)
            return w;
    }
    return 0;
}

bool overlaps(const void* a, int64_t an, const void* b, int64_t bn)
{
    if (an <= 0 || bn <= 0)
        return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + uint64_t(bn) && b0 < a0 + uint64_t(an);
}

// Byte extent of a strided tensor (non-negative element strides, esize bytes).
bool extent(std::initializer_list<int64_t> dims, std::initializer_list<int64_t> strides,
            int64_t esize, int64_t* out)
{
    int64_t last = 0;
    auto s = strides.begin();
    for (int64_t n : dims) {
        if (n == 0) {
            *out = 0;
            return true;
        }
        int64_t term;
        if (!mul_ok(n - 1, *s, &term) || last > kI64Max - term)
            return false;
        last += term;
        ++s;
    }
    if (last == kI64Max)
        return false;
    return mul_ok(last + 1, esize, out);
}

uint32_t pow2ceil(uint32_t x)
{
    uint32_t p = 1;
    while (p < x)
        p <<= 1;
    return p;
}

uint32_t log2u(uint32_t x)
{
    uint32_t l = 0;
    while ((1u << l) < x)
        ++l;
    return l;
}

constexpr uint64_t kU32Limit = (uint64_t(1) << 31);  // vector-index headroom inside one slab

uint32_t tiles(uint64_t vecs, uint64_t per_tile) { return uint32_t((vecs + per_tile - 1) / per_tile); }

// ---------------------------------------------------------------- relayouts

cam_status dense_relayout(const void* in, void* out, int64_t P, int64_t B, int64_t S, int64_t H,
                          int64_t D, cam_dtype dt, void* stream, bool seq_to_head)
{
    const char* op = seq_to_head ? "ulysses_seq_to_head" : "ulysses_head_to_seq";
    clear_error();
    if (P < 1 || B < 0 || S < 0 || H < 0 || D < 0)
        return set_error(CAM_ERR_SHAPE, "%s: need P >= 1 and B, S, H, D >= 0 (P=%lld B=%lld S=%lld H=%lld D=%lld)",
                         op, (long long)P, (long long)B, (long long)S, (long long)H, (long long)D);
    const int es = elem_size(dt);
    if (!es)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: unknown dtype code %d", op, int(dt));
    if (S % P || H % P)
        return set_error(CAM_ERR_DIVISIBILITY, "%s: S (%lld) and H (%lld) must be multiples of P (%lld)",
                         op, (long long)S, (long long)H, (long long)P);
    int64_t bytes;
    if (!prod_ok({B, S, H, D, es}, &bytes))
        return set_error(CAM_ERR_SHAPE, "%s: B*S*H*D*esize overflows", op);
    if (bytes == 0)
        return CAM_OK;
    if (!in || !out)
        return set_error(CAM_ERR_NULL, "%s: in and out must be non-null", op);
    if (!aligned(in, es) || !aligned(out, es))
        return set_error(CAM_ERR_ALIGNMENT, "%s: pointers must be aligned to the %s element size", op, dt_name(dt));
    if (overlaps(in, bytes, out, bytes))
        return set_error(CAM_ERR_OVERLAP, "%s: in and out overlap", op);
    if (P > UINT32_MAX || B > UINT32_MAX)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: P and B must fit 32 bits", op);

    const uint64_t run = uint64_t(H / P) * uint64_t(D) * es;
    DenseRelayout a{};
    a.width = pick_width({run, reinterpret_cast<uintptr_t>(in), reinterpret_cast<uintptr_t>(out)});
    if (run / a.width >= kU32Limit)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: one head block of one row exceeds 2^31 vectors", op);
    a.src = in;
    a.dst = out;
    a.P = uint32_t(P);
    a.B = uint32_t(B);
    a.div_P = make_fastdiv(a.P);
    a.div_B = make_fastdiv(a.B);
    a.c = uint32_t(run / a.width);
    a.div_c = make_fastdiv(a.c);
    a.Pc = uint64_t(P) * a.c;
    a.Sp = uint64_t(S / P);
    const uint64_t slab_vecs = a.Sp * a.c;
    if (slab_vecs >= kU32Limit)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: one (rank, plane, rank) slab exceeds 2^31 vectors", op);
    a.slab_vecs = uint32_t(slab_vecs);
    a.tiles_per_slab = tiles(slab_vecs, kDenseTileVecs);
    a.div_tps = make_fastdiv(a.tiles_per_slab);
    const uint64_t n_tiles = uint64_t(P) * uint64_t(B) * uint64_t(P) * a.tiles_per_slab;
    if (n_tiles > UINT32_MAX)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: more than 2^32 tiles", op);
    a.n_tiles = uint32_t(n_tiles);
    a.seq_to_head = seq_to_head;
    return launch_dense_relayout(a, stream);
}

// LDS-staged seq->head (ablation): 16-byte accesses only, R rows per tile
// staged whole in LDS (at most 64 KiB and 256 * 24 vectors per tile).
cam_status ablation_seq_to_head_lds(const void* in, void* out, int64_t P, int64_t B, int64_t S, int64_t H,
                                    int64_t D, cam_dtype dt, int64_t R, void* stream)
{
    const char* op = "cam_ablation_seq_to_head_lds";
    clear_error();
    if (P < 1 || B < 0 || S < 0 || H < 0 || D < 0)
        return set_error(CAM_ERR_SHAPE, "%s: need P >= 1 and B, S, H, D >= 0", op);
    const int es = elem_size(dt);
    if (!es)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: unknown dtype code %d", op, int(dt));
    if (S % P || H % P)
        return set_error(CAM_ERR_DIVISIBILITY, "%s: S and H must be multiples of P", op);
    int64_t bytes;
    if (!prod_ok({B, S, H, D, es}, &bytes))
        return set_error(CAM_ERR_SHAPE, "%s: B*S*H*D*esize overflows", op);
    if (bytes == 0)
        return CAM_OK;
    if (!in || !out)
        return set_error(CAM_ERR_NULL, "%s: in and out must be non-null", op);
    const uint64_t run = uint64_t(H / P) * uint64_t(D) * es;
    if (run % 16 || !aligned(in, 16) || !aligned(out, 16))
        return set_error(CAM_ERR_ALIGNMENT, "%s: 16-byte accesses only: runs and pointers must be 16-byte multiples",
                         op);
    if (overlaps(in, bytes, out, bytes))
        return set_error(CAM_ERR_OVERLAP, "%s: in and out overlap", op);
    const uint64_t c = run / 16;
    if (R < 1 || R > 4096 || P > 4096 || B > int64_t(UINT32_MAX) || uint64_t(R) * uint64_t(P) * c > 4096)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: rows_per_tile * H * D * esize must be within 64 KiB of LDS", op);
    DenseLds a{};
    a.src = in;
    a.dst = out;
    a.P = uint32_t(P);
    a.B = uint32_t(B);
    a.c = uint32_t(c);
    a.div_c = make_fastdiv(a.c);
    a.R = uint32_t(R);
    a.Rc = uint32_t(R * c);
    a.div_Rc = make_fastdiv(a.Rc);
    a.Sp = uint64_t(S / P);
    const uint64_t tps = (a.Sp + a.R - 1) / a.R;
    const uint64_t n_tiles = uint64_t(P) * uint64_t(B) * tps;
    if (n_tiles > UINT32_MAX || a.Sp * uint64_t(P) * c * uint64_t(B) * uint64_t(P) >= (uint64_t(1) << 40))
        return set_error(CAM_ERR_UNSUPPORTED, "%s: too many tiles", op);
    a.tiles_per_slab = uint32_t(tps);
    a.div_tps = make_fastdiv(a.tiles_per_slab);
    a.div_B = make_fastdiv(a.B);
    a.n_tiles = uint32_t(n_tiles);
    return launch_dense_lds(a, stream);
}

// The per-sequence split (rank_cu, rank_off from ulysses_varlen_plan), or with
// span_rank non-null a THD layout plan: cu = span starts, nseq = span count,
// span_rank / span_local / rank_off from thd_plan.
cam_status varlen_relayout(const void* in, void* out, const int32_t* cu, const int32_t* rank_cu,
                           const int64_t* rank_off, int64_t nseq, int64_t T, int64_t P, int64_t B,
                           int64_t H, int64_t D, cam_dtype dt, void* stream, bool seq_to_head,
                           const int32_t* span_rank = nullptr, const int32_t* span_local = nullptr)
{
    const bool spans = span_rank != nullptr || span_local != nullptr;
    const char* op = spans ? (seq_to_head ? "ulysses_seq_to_head_spans" : "ulysses_head_to_seq_spans")
                           : (seq_to_head ? "ulysses_seq_to_head_varlen" : "ulysses_head_to_seq_varlen");
    clear_error();
    if (P < 1 || B < 0 || T < 0 || H < 0 || D < 0 || nseq < 0)
        return set_error(CAM_ERR_SHAPE, "%s: need P >= 1 and nseq, total_tokens, B, H, D >= 0", op);
    const int es = elem_size(dt);
    if (!es)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: unknown dtype code %d", op, int(dt));
    if (H % P)
        return set_error(CAM_ERR_DIVISIBILITY, "%s: H (%lld) must be a multiple of P (%lld)", op,
                         (long long)H, (long long)P);
    if (T > INT32_MAX || nseq >= INT32_MAX)
        return set_error(CAM_ERR_SHAPE, "%s: total_tokens and nseq must fit int32 (cu_seqlens is int32)", op);
    if (T > 0 && nseq < 1)
        return set_error(CAM_ERR_SHAPE, "%s: total_tokens > 0 needs nseq >= 1", op);
    int64_t bytes;
    if (!prod_ok({B, T, H, D, es}, &bytes))
        return set_error(CAM_ERR_SHAPE, "%s: B*T*H*D*esize overflows", op);
    if (bytes == 0)
        return CAM_OK;
    if (spans) {
        if (!in || !out || !cu || !span_rank || !span_local || !rank_off)
            return set_error(CAM_ERR_NULL, "%s: in, out, span_start, span_rank, span_local and rank_off must be "
                                           "non-null", op);
        if (!aligned(in, es) || !aligned(out, es) || !aligned(cu, 4) || !aligned(span_rank, 4) ||
            !aligned(span_local, 4) || !aligned(rank_off, 8))
            return set_error(CAM_ERR_ALIGNMENT, "%s: misaligned pointer", op);
        if (overlaps(in, bytes, out, bytes))
            return set_error(CAM_ERR_OVERLAP, "%s: in and out overlap", op);
        if (overlaps(out, bytes, cu, 4 * (nseq + 1)) || overlaps(out, bytes, span_rank, 4 * nseq) ||
            overlaps(out, bytes, span_local, 4 * nseq) || overlaps(out, bytes, rank_off, 8 * (P + 1)))
            return set_error(CAM_ERR_OVERLAP, "%s: out overlaps the plan arrays", op);
    } else {
        if (!in || !out || !cu || !rank_cu || !rank_off)
            return set_error(CAM_ERR_NULL, "%s: in, out, cu_seqlens, rank_cu and rank_off must be non-null", op);
        if (!aligned(in, es) || !aligned(out, es) || !aligned(cu, 4) || !aligned(rank_cu, 4) ||
            !aligned(rank_off, 8))
            return set_error(CAM_ERR_ALIGNMENT, "%s: misaligned pointer", op);
        if (overlaps(in, bytes, out, bytes))
            return set_error(CAM_ERR_OVERLAP, "%s: in and out overlap", op);
        if (overlaps(out, bytes, cu, 4 * (nseq + 1)) || overlaps(out, bytes, rank_cu, 4 * P * (nseq + 1)) ||
            overlaps(out, bytes, rank_off, 8 * (P + 1)))
            return set_error(CAM_ERR_OVERLAP, "%s: out overlaps the plan arrays", op);
    }
    if (P > UINT32_MAX || B > UINT32_MAX)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: P and B must fit 32 bits", op);

    const uint64_t run = uint64_t(H / P) * uint64_t(D) * es;
    VarlenRelayout a{};
    a.width = pick_width({run, reinterpret_cast<uintptr_t>(in), reinterpret_cast<uintptr_t>(out)});
    if (run / a.width >= kU32Limit)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: one head block of one row exceeds 2^31 vectors", op);
    a.src = in;
    a.dst = out;
    a.cu = cu;
    a.rank_cu = rank_cu;
    a.rank_off = rank_off;
    a.span_rank = span_rank;
    a.span_local = span_local;
    a.spans = spans;
    a.nseq = int32_t(nseq);
    a.P = uint32_t(P);
    a.B = uint32_t(B);
    a.div_P = make_fastdiv(a.P);
    a.div_B = make_fastdiv(a.B);
    a.T = uint64_t(T);
    a.c = uint32_t(run / a.width);
    a.div_c = make_fastdiv(a.c);
    a.Pc = uint64_t(P) * a.c;
    a.plane_vecs = uint64_t(T) * a.c;
    if (a.plane_vecs >= kU32Limit)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: one (rank, plane) exceeds 2^31 vectors", op);
    a.tiles_per_plane = tiles(a.plane_vecs, kVarlenTileVecs);
    a.div_tpp = make_fastdiv(a.tiles_per_plane);
    const uint64_t n_tiles = uint64_t(P) * uint64_t(B) * a.tiles_per_plane;
    if (n_tiles > UINT32_MAX)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: more than 2^32 tiles", op);
    a.n_tiles = uint32_t(n_tiles);
    a.seq_to_head = seq_to_head;
    return launch_varlen_relayout(a, stream);
}

// --------------------------------------------------------------------- pack

struct PackGeom {
    int64_t rows, o_region, chunk, total;
};

cam_status pack_geometry(const char* op, int64_t P, int64_t T, int64_t H, int64_t Dv, int scatter_dim,
                         cam_dtype dt, PackGeom* g)
{
    if (P < 1 || T < 0 || H < 0 || Dv < 0)
        return set_error(CAM_ERR_SHAPE, "%s: need P >= 1 and T, H, Dv >= 0", op);
    if (dt != CAM_BF16 && dt != CAM_FP16)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: payload dtype must be bf16 or fp16", op);
    if (scatter_dim != 0 && scatter_dim != 1)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: scatter_dim must be 0 (tokens) or 1 (heads)", op);
    if (scatter_dim == 1 && H % P)
        return set_error(CAM_ERR_DIVISIBILITY, "%s: scatter_dim 1 needs H %% P == 0 (H=%lld P=%lld)", op,
                         (long long)H, (long long)P);
    if (scatter_dim == 0 && T % P)
        return set_error(CAM_ERR_DIVISIBILITY, "%s: scatter_dim 0 needs T %% P == 0 (T=%lld P=%lld)", op,
                         (long long)T, (long long)P);
    int64_t rows, obytes, lbytes, chunk, total;
    if (!prod_ok({scatter_dim == 1 ? T : T / P, scatter_dim == 1 ? H / P : H}, &rows) ||
        !prod_ok({rows, Dv, 2}, &obytes) || obytes > kI64Max / 4 || !prod_ok({rows, 4}, &lbytes) ||
        lbytes > kI64Max / 4)
        return set_error(CAM_ERR_SHAPE, "%s: sizes overflow", op);
    obytes = (obytes + 15) / 16 * 16;
    chunk = obytes + (lbytes + 15) / 16 * 16;  // each term below 2^61: no overflow
    if (!prod_ok({P, P, chunk}, &total))
        return set_error(CAM_ERR_SHAPE, "%s: packed size overflows", op);
    g->rows = rows;
    g->o_region = obytes;
    g->chunk = chunk;
    g->total = total;
    return CAM_OK;
}

struct CombineIn {
    const void* po;
    int64_t po_sp, po_st, po_sh;  // elements
    const float* pl;
    int64_t pl_sp, pl_st, pl_sh;  // elements
    int64_t P, T, H, D;
    cam_dtype dt;
    void* out;
    int64_t o_st, o_sh;           // elements
    float* lse_out;
    int64_t lo_st, lo_sh;
    const int32_t* cu;
    int64_t nseq;
    uint32_t out_mode = 0;           // see Combine::out_mode
    int64_t Hp = 0, Hq = 0;          // mode 1
    const int32_t* rank_cu = nullptr;  // mode 2
    const int64_t* rank_off = nullptr;
    const int32_t* first = nullptr;    // a plan's first positions [P][nseq] (planned rule)
};

cam_status combine(const char* op, const CombineIn& c, void* stream)
{
    if (c.P < 1 || c.T < 0 || c.H < 0 || c.D < 0)
        return set_error(CAM_ERR_SHAPE, "%s: need P >= 1 and T, H, D >= 0", op);
    if (c.P > 64)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: at most 64 partials per row (P=%lld)", op, (long long)c.P);
    if (c.dt != CAM_BF16 && c.dt != CAM_FP16)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: payload dtype must be bf16 or fp16", op);
    for (int64_t s : {c.po_sp, c.po_st, c.po_sh, c.pl_sp, c.pl_st, c.pl_sh, c.o_st, c.o_sh, c.lo_st, c.lo_sh})
        if (s < 0 || s > kMaxStride)
            return set_error(CAM_ERR_UNSUPPORTED, "%s: strides must be non-negative and below 2^48", op);
    int64_t n_rows;
    if (!prod_ok({c.T, c.H}, &n_rows))
        return set_error(CAM_ERR_SHAPE, "%s: T*H overflows", op);
    if (n_rows == 0)
        return CAM_OK;
    if (n_rows > INT32_MAX)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: T*H must be below 2^31 rows", op);
    if (c.cu && c.nseq < 1)
        return set_error(CAM_ERR_SHAPE, "%s: nseq must be >= 1", op);
    if (c.cu && c.T > INT32_MAX)
        return set_error(CAM_ERR_SHAPE, "%s: total_tokens must fit int32", op);
    if (!c.po || !c.pl || !c.out)
        return set_error(CAM_ERR_NULL, "%s: partial outputs, partial LSEs and out must be non-null", op);
    if (!aligned(c.po, 2) || !aligned(c.pl, 4) || !aligned(c.out, 2) || (c.lse_out && !aligned(c.lse_out, 4)) ||
        (c.cu && !aligned(c.cu, 4)))
        return set_error(CAM_ERR_ALIGNMENT, "%s: misaligned pointer", op);
    int64_t ext_po, ext_pl, ext_o, ext_lo = 0;
    if (!extent({c.P, c.T, c.H, c.D}, {c.po_sp, c.po_st, c.po_sh, 1}, 2, &ext_po) ||
        !extent({c.P, c.T, c.H}, {c.pl_sp, c.pl_st, c.pl_sh}, 4, &ext_pl) ||
        !extent({c.T, c.H, c.D}, {c.o_st, c.o_sh, 1}, 2, &ext_o) ||
        (c.lse_out && !extent({c.T, c.H}, {c.lo_st, c.lo_sh}, 4, &ext_lo)))
        return set_error(CAM_ERR_SHAPE, "%s: tensor extent overflows", op);
    if (overlaps(c.out, ext_o, c.po, ext_po) || overlaps(c.out, ext_o, c.pl, ext_pl) ||
        overlaps(c.lse_out, ext_lo, c.po, ext_po) || overlaps(c.lse_out, ext_lo, c.pl, ext_pl) ||
        overlaps(c.out, ext_o, c.lse_out, ext_lo))
        return set_error(CAM_ERR_OVERLAP, "%s: an output overlaps an input or the other output", op);
    if (c.cu && (overlaps(c.out, ext_o, c.cu, 4 * (c.nseq + 1)) || overlaps(c.lse_out, ext_lo, c.cu, 4 * (c.nseq + 1))))
        return set_error(CAM_ERR_OVERLAP, "%s: an output overlaps cu_seqlens", op);
    if (c.first) {
        int64_t ext_f;
        if (!c.cu || !prod_ok({c.P, c.nseq, 4}, &ext_f))
            return set_error(CAM_ERR_SHAPE, "%s: the first-position table needs cu_seqlens", op);
        if (!aligned(c.first, 4))
            return set_error(CAM_ERR_ALIGNMENT, "%s: misaligned first-position table", op);
        if (overlaps(c.out, ext_o, c.first, ext_f) || overlaps(c.lse_out, ext_lo, c.first, ext_f))
            return set_error(CAM_ERR_OVERLAP, "%s: an output overlaps the first-position table", op);
    }

    Combine a{};
    const uint64_t row_b = uint64_t(c.D) * 2;
    a.width = pick_width({row_b == 0 ? 16 : row_b, reinterpret_cast<uintptr_t>(c.po), reinterpret_cast<uintptr_t>(c.out),
                          uint64_t(c.po_sp) * 2, uint64_t(c.po_st) * 2, uint64_t(c.po_sh) * 2,
                          uint64_t(c.o_st) * 2, uint64_t(c.o_sh) * 2});
    a.po = c.po;
    a.po_sp_b = c.po_sp * 2;
    a.po_st_b = c.po_st * 2;
    a.po_sh_b = c.po_sh * 2;
    a.pl = c.pl;
    a.pl_sp = c.pl_sp;
    a.pl_st = c.pl_st;
    a.pl_sh = c.pl_sh;
    a.out = c.out;
    a.o_st_b = c.o_st * 2;
    a.o_sh_b = c.o_sh * 2;
    a.lse_out = c.lse_out;
    a.lo_st = c.lo_st;
    a.lo_sh = c.lo_sh;
    a.P = uint32_t(c.P);
    a.H = uint32_t(c.H);
    a.div_H = make_fastdiv(a.H);
    a.n_rows = uint64_t(n_rows);
    if (row_b / a.width >= kU32Limit)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: one row exceeds 2^31 vectors", op);
    a.cv = uint32_t(row_b / a.width);
    a.g_log2 = log2u(pow2ceil(a.cv < 64 ? (a.cv ? a.cv : 1) : 64));
    if (a.g_log2 < 6 && kCombineNarrowVpl == 2 && a.g_log2 > 0)
        a.g_log2 -= 1;  // narrow rows: each lane moves two vectors of the row per pass
    a.gp_log2 = log2u(pow2ceil(a.P));
    // tile geometry (measured per row width): rows per tile, workgroup size,
    // tile order; at least one row per payload group
    const bool wave = a.g_log2 == 6;
    a.xcd = wave ? CAM_XCD_COMBINE_WAVE : CAM_XCD_COMBINE_NARROW;
    uint32_t rows = wave                                   ? CAM_COMBINE_ROWS_WAVE
                    : uint64_t(a.cv) * a.width >= 512 ? CAM_COMBINE_ROWS_WIDE
                                                      : CAM_COMBINE_ROWS_NARROW;
    // a workgroup holds one lane group per row of its tile (64 to 256
    // threads), so very short rows take a smaller workgroup rather than a
    // larger tile: the tile's per-row tables in LDS stay within 64 KiB
    a.threads = wave ? CAM_COMBINE_THREADS_WAVE
                     : std::min<uint32_t>(kThreads, std::max<uint32_t>(64u, rows << a.g_log2));
    const uint32_t groups = a.threads >> a.g_log2;
    if (rows < groups)
        rows = groups;
    if (!wave) {
        // many partials: the first phase gives every (row, partial) a lane, so
        // a tile takes (rows * pow2(P)) / threads dependent rounds of LSE
        // loads; widen the workgroup, then shorten the tile, to cap them
        const auto rounds = [&] { return (uint64_t(rows) << a.gp_log2) / a.threads; };
        while (rounds() > CAM_COMBINE_STATS_ROUNDS && a.threads < kThreads)
            a.threads *= 2;
        while (rounds() > CAM_COMBINE_STATS_ROUNDS && rows > 1)
            rows /= 2;
    }
    a.rows_per_tile = rows;
    a.n_tiles = (uint64_t(n_rows) + rows - 1) / rows;
    a.cu = c.cu;
    a.nseq = int32_t(c.nseq);
    a.div_P = make_fastdiv(a.P);
    a.out_mode = c.out_mode;
    a.Hp = uint32_t(c.Hp);
    a.Hq = uint32_t(c.Hq);
    a.div_Hp = make_fastdiv(c.Hp > 0 ? uint32_t(c.Hp) : 1u);
    a.o_row_b = uint64_t(c.D) * 2;
    a.rank_cu = c.rank_cu;
    a.rank_off = c.rank_off;
    a.first = c.first;
    a.fp16 = c.dt == CAM_FP16;
    return launch_combine(a, stream);
}

struct CombineBwdIn {
    const void* po;
    int64_t po_sp, po_st, po_sh;
    const float* pl;
    int64_t pl_sp, pl_st, pl_sh;
    int64_t P, T, H, D;
    cam_dtype dt;
    const void* go;
    int64_t go_st, go_sh;
    const float* gl;
    int64_t gl_st, gl_sh;
    void* dpo;
    int64_t dpo_sp, dpo_st, dpo_sh;
    float* dpl;
    int64_t dpl_sp, dpl_st, dpl_sh;
    const int32_t* cu;
    int64_t nseq;
    const int32_t* first = nullptr;  // a plan's first positions [P][nseq] (planned rule)
};

cam_status combine_backward(const char* op, const CombineBwdIn& c, void* stream)
{
    if (c.P < 1 || c.T < 0 || c.H < 0 || c.D < 0)
        return set_error(CAM_ERR_SHAPE, "%s: need P >= 1 and T, H, D >= 0", op);
    if (c.P > 64)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: at most 64 partials per row (P=%lld)", op, (long long)c.P);
    if (c.dt != CAM_BF16 && c.dt != CAM_FP16)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: payload dtype must be bf16 or fp16", op);
    for (int64_t s : {c.po_sp, c.po_st, c.po_sh, c.pl_sp, c.pl_st, c.pl_sh, c.go_st, c.go_sh, c.gl_st, c.gl_sh,
                      c.dpo_sp, c.dpo_st, c.dpo_sh, c.dpl_sp, c.dpl_st, c.dpl_sh})
        if (s < 0 || s > kMaxStride)
            return set_error(CAM_ERR_UNSUPPORTED, "%s: strides must be non-negative and below 2^48", op);
    int64_t n_rows;
    if (!prod_ok({c.T, c.H}, &n_rows))
        return set_error(CAM_ERR_SHAPE, "%s: T*H overflows", op);
    if (n_rows == 0)
        return CAM_OK;
    if (n_rows > INT32_MAX)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: T*H must be below 2^31 rows", op);
    if (c.cu && c.nseq < 1)
        return set_error(CAM_ERR_SHAPE, "%s: nseq must be >= 1", op);
    if (!c.po || !c.pl || !c.go || !c.dpo || !c.dpl)
        return set_error(CAM_ERR_NULL, "%s: partials, their LSEs, the output gradient and both input "
                                       "gradients must be non-null", op);
    if (!aligned(c.po, 2) || !aligned(c.pl, 4) || !aligned(c.go, 2) || (c.gl && !aligned(c.gl, 4)) ||
        !aligned(c.dpo, 2) || !aligned(c.dpl, 4) || (c.cu && !aligned(c.cu, 4)))
        return set_error(CAM_ERR_ALIGNMENT, "%s: misaligned pointer", op);
    int64_t ext_po, ext_pl, ext_go, ext_gl = 0, ext_dpo, ext_dpl;
    if (!extent({c.P, c.T, c.H, c.D}, {c.po_sp, c.po_st, c.po_sh, 1}, 2, &ext_po) ||
        !extent({c.P, c.T, c.H}, {c.pl_sp, c.pl_st, c.pl_sh}, 4, &ext_pl) ||
        !extent({c.T, c.H, c.D}, {c.go_st, c.go_sh, 1}, 2, &ext_go) ||
        (c.gl && !extent({c.T, c.H}, {c.gl_st, c.gl_sh}, 4, &ext_gl)) ||
        !extent({c.P, c.T, c.H, c.D}, {c.dpo_sp, c.dpo_st, c.dpo_sh, 1}, 2, &ext_dpo) ||
        !extent({c.P, c.T, c.H}, {c.dpl_sp, c.dpl_st, c.dpl_sh}, 4, &ext_dpl))
        return set_error(CAM_ERR_SHAPE, "%s: tensor extent overflows", op);
    const int64_t ext_cu = c.cu ? 4 * (c.nseq + 1) : 0;
    for (auto out : {std::make_pair(static_cast<const void*>(c.dpo), ext_dpo),
                     std::make_pair(static_cast<const void*>(c.dpl), ext_dpl)})
        if (overlaps(out.first, out.second, c.po, ext_po) || overlaps(out.first, out.second, c.pl, ext_pl) ||
            overlaps(out.first, out.second, c.go, ext_go) || overlaps(out.first, out.second, c.gl, ext_gl) ||
            overlaps(out.first, out.second, c.cu, ext_cu))
            return set_error(CAM_ERR_OVERLAP, "%s: an output overlaps an input", op);
    if (overlaps(c.dpo, ext_dpo, c.dpl, ext_dpl))
        return set_error(CAM_ERR_OVERLAP, "%s: the two outputs overlap", op);
    if (c.first) {
        int64_t ext_f;
        if (!c.cu || !prod_ok({c.P, c.nseq, 4}, &ext_f))
            return set_error(CAM_ERR_SHAPE, "%s: the first-position table needs cu_seqlens", op);
        if (!aligned(c.first, 4))
            return set_error(CAM_ERR_ALIGNMENT, "%s: misaligned first-position table", op);
        if (overlaps(c.dpo, ext_dpo, c.first, ext_f) || overlaps(c.dpl, ext_dpl, c.first, ext_f))
            return set_error(CAM_ERR_OVERLAP, "%s: an output overlaps the first-position table", op);
    }

    CombineBwd a{};
    const uint64_t row_b = uint64_t(c.D) * 2;
    a.width = pick_width({row_b == 0 ? 16 : row_b, reinterpret_cast<uintptr_t>(c.po), reinterpret_cast<uintptr_t>(c.go),
                          reinterpret_cast<uintptr_t>(c.dpo), uint64_t(c.po_sp) * 2, uint64_t(c.po_st) * 2,
                          uint64_t(c.po_sh) * 2, uint64_t(c.go_st) * 2, uint64_t(c.go_sh) * 2,
                          uint64_t(c.dpo_sp) * 2, uint64_t(c.dpo_st) * 2, uint64_t(c.dpo_sh) * 2});
    a.po = c.po;
    a.po_sp_b = c.po_sp * 2;
    a.po_st_b = c.po_st * 2;
    a.po_sh_b = c.po_sh * 2;
    a.pl = c.pl;
    a.pl_sp = c.pl_sp;
    a.pl_st = c.pl_st;
    a.pl_sh = c.pl_sh;
    a.go = c.go;
    a.go_st_b = c.go_st * 2;
    a.go_sh_b = c.go_sh * 2;
    a.gl = c.gl;
    a.gl_st = c.gl_st;
    a.gl_sh = c.gl_sh;
    a.dpo = c.dpo;
    a.dpo_sp_b = c.dpo_sp * 2;
    a.dpo_st_b = c.dpo_st * 2;
    a.dpo_sh_b = c.dpo_sh * 2;
    a.dpl = c.dpl;
    a.dpl_sp = c.dpl_sp;
    a.dpl_st = c.dpl_st;
    a.dpl_sh = c.dpl_sh;
    a.P = uint32_t(c.P);
    a.H = uint32_t(c.H);
    a.div_H = make_fastdiv(a.H);
    a.n_rows = uint64_t(n_rows);
    if (row_b / a.width >= kU32Limit)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: one row exceeds 2^31 vectors", op);
    a.cv = uint32_t(row_b / a.width);
    a.gp_log2 = log2u(pow2ceil(a.P));
    const uint32_t g_full = log2u(pow2ceil(a.cv < 64 ? (a.cv ? a.cv : 1) : 64));
    const uint32_t rows0 = uint64_t(a.cv) * a.width >= 512 ? CAM_COMBINE_BWD_ROWS_WIDE : CAM_COMBINE_BWD_ROWS_NARROW;
    // compacted form: each lane moves kCombineBwdVpl vectors of a row per
    // pass, the workgroup holds one lane group per row of its tile, and the
    // per-lane dot products of every (row, valid partial) are reduced in LDS;
    // used when those tables fit 64 KiB, otherwise the row groups reduce with
    // cross-lane shuffles
    {
        const uint32_t g = (kCombineBwdVpl == 2 && g_full > 0 && g_full < 6) ? g_full - 1 : g_full;
        uint32_t threads = std::min<uint32_t>(kThreads, std::max<uint32_t>(64u, rows0 << g));
        uint32_t rows = std::max(rows0, threads >> g);
        // many partials: cap the first phase's rounds as the forward does
        while ((uint64_t(rows) << a.gp_log2) / threads > CAM_COMBINE_STATS_ROUNDS && threads < kThreads)
            threads *= 2;
        while ((uint64_t(rows) << a.gp_log2) / threads > CAM_COMBINE_STATS_ROUNDS && rows > 1)
            rows /= 2;
        const uint64_t lds = uint64_t(rows) * a.P * (4 + 8 + 4 * (uint64_t(1) << g)) + uint64_t(rows) * (8 + 4 + 4) +
                             (c.cu && c.nseq < kCuCache ? uint64_t(c.nseq + 1) * 4 : 0) + 16;
        a.compact = g_full < 6 && lds <= 65536;
        if (a.compact) {
            a.g_log2 = g;
            a.threads = threads;
            a.rows_per_tile = rows;
        }
    }
    if (!a.compact) {
        a.g_log2 = g_full;
        a.threads = kThreads;
        a.rows_per_tile = std::max(rows0, uint32_t(kThreads) >> g_full);
    }
    const uint32_t rows = a.rows_per_tile;
    a.n_tiles = (uint64_t(n_rows) + rows - 1) / rows;
    a.cu = c.cu;
    a.first = c.first;
    a.nseq = int32_t(c.nseq);
    a.div_P = make_fastdiv(a.P);
    a.fp16 = c.dt == CAM_FP16;
    return launch_combine_bwd(a, stream);
}

}  // namespace
}  // namespace cam

using namespace cam;

extern "C" {

const char* cam_status_string(cam_status s)
{
    switch (s) {
    case CAM_OK: return "CAM_OK";
    case CAM_ERR_NULL: return "CAM_ERR_NULL";
    case CAM_ERR_SHAPE: return "CAM_ERR_SHAPE";
    case CAM_ERR_DIVISIBILITY: return "CAM_ERR_DIVISIBILITY";
    case CAM_ERR_ALIGNMENT: return "CAM_ERR_ALIGNMENT";
    case CAM_ERR_OVERLAP: return "CAM_ERR_OVERLAP";
    case CAM_ERR_UNSUPPORTED: return "CAM_ERR_UNSUPPORTED";
    case CAM_ERR_HIP: return "CAM_ERR_HIP";
    }
    return "CAM_ERR_UNKNOWN";
}

const char* cam_last_error(void) { return g_err; }

cam_status cam_last_launch(uint64_t* workgroups, uint32_t* threads, uint64_t* lds_bytes)
{
    if (!workgroups || !threads || !lds_bytes)
        return set_error(CAM_ERR_NULL, "cam_last_launch: null output pointer");
    *workgroups = g_launch[0];
    *threads = uint32_t(g_launch[1]);
    *lds_bytes = g_launch[2];
    return CAM_OK;
}

int cam_abi_version(void) { return CAM_ABI_VERSION; }

cam_status ulysses_seq_to_head(const void* in, void* out, int64_t P, int64_t B, int64_t S, int64_t H,
                               int64_t D, cam_dtype dt, void* stream)
{
    return dense_relayout(in, out, P, B, S, H, D, dt, stream, true);
}

cam_status ulysses_head_to_seq(const void* in, void* out, int64_t P, int64_t B, int64_t S, int64_t H,
                               int64_t D, cam_dtype dt, void* stream)
{
    return dense_relayout(in, out, P, B, S, H, D, dt, stream, false);
}

cam_status cam_ablation_seq_to_head_lds(const void* in, void* out, int64_t P, int64_t B, int64_t S, int64_t H,
                                        int64_t D, cam_dtype dt, int64_t rows_per_tile, void* stream)
{
    return ablation_seq_to_head_lds(in, out, P, B, S, H, D, dt, rows_per_tile, stream);
}

cam_status ulysses_seq_to_head_spans(const void* in, void* out, const int32_t* span_start, const int32_t* span_rank,
                                     const int32_t* span_local, const int64_t* rank_off, int64_t n_spans,
                                     int64_t total_tokens, int64_t P, int64_t B, int64_t H, int64_t D, cam_dtype dt,
                                     void* stream)
{
    if (total_tokens > 0 && (!span_rank || !span_local))
        return set_error(CAM_ERR_NULL, "ulysses_seq_to_head_spans: span_rank and span_local must be non-null");
    return varlen_relayout(in, out, span_start, nullptr, rank_off, n_spans, total_tokens, P, B, H, D, dt, stream,
                           true, span_rank, span_local);
}

cam_status ulysses_head_to_seq_spans(const void* in, void* out, const int32_t* span_start, const int32_t* span_rank,
                                     const int32_t* span_local, const int64_t* rank_off, int64_t n_spans,
                                     int64_t total_tokens, int64_t P, int64_t B, int64_t H, int64_t D, cam_dtype dt,
                                     void* stream)
{
    if (total_tokens > 0 && (!span_rank || !span_local))
        return set_error(CAM_ERR_NULL, "ulysses_head_to_seq_spans: span_rank and span_local must be non-null");
    return varlen_relayout(in, out, span_start, nullptr, rank_off, n_spans, total_tokens, P, B, H, D, dt, stream,
                           false, span_rank, span_local);
}

cam_status ulysses_varlen_plan(const int32_t* cu, int64_t nseq, int64_t P, int32_t* rank_cu,
                               int64_t* rank_off)
{
    clear_error();
    if (P < 1 || nseq < 0)
        return set_error(CAM_ERR_SHAPE, "ulysses_varlen_plan: need P >= 1 and nseq >= 0");
    if (!cu || !rank_cu || !rank_off)
        return set_error(CAM_ERR_NULL, "ulysses_varlen_plan: cu_seqlens, rank_cu and rank_off must be non-null");
    if (cu[0] != 0)
        return set_error(CAM_ERR_SHAPE, "ulysses_varlen_plan: cu_seqlens[0] must be 0 (got %d)", cu[0]);
    for (int64_t i = 0; i < nseq; ++i)
        if (cu[i + 1] < cu[i])
            return set_error(CAM_ERR_SHAPE, "ulysses_varlen_plan: cu_seqlens decreases at %lld", (long long)i);
    // Sizes of the pieces of sequence i on rank p: floor((p+1)L/P) - floor(pL/P).
    int64_t off = 0;
    for (int64_t p = 0; p < P; ++p) {
        rank_off[p] = off;
        int64_t run = 0;
        for (int64_t i = 0; i < nseq; ++i) {
            rank_cu[p * (nseq + 1) + i] = int32_t(run);
            const int64_t L = int64_t(cu[i + 1]) - cu[i];
            run += (p + 1) * L / P - p * L / P;
        }
        rank_cu[p * (nseq + 1) + nseq] = int32_t(run);
        off += run;
    }
    rank_off[P] = off;
    return CAM_OK;
}

cam_status ulysses_seq_to_head_varlen(const void* in, void* out, const int32_t* cu, const int32_t* rank_cu,
                                      const int64_t* rank_off, int64_t nseq, int64_t total_tokens, int64_t P,
                                      int64_t B, int64_t H, int64_t D, cam_dtype dt, void* stream)
{
    return varlen_relayout(in, out, cu, rank_cu, rank_off, nseq, total_tokens, P, B, H, D, dt, stream, true);
}

cam_status ulysses_head_to_seq_varlen(const void* in, void* out, const int32_t* cu, const int32_t* rank_cu,
                                      const int64_t* rank_off, int64_t nseq, int64_t total_tokens, int64_t P,
                                      int64_t B, int64_t H, int64_t D, cam_dtype dt, void* stream)
{
    return varlen_relayout(in, out, cu, rank_cu, rank_off, nseq, total_tokens, P, B, H, D, dt, stream, false);
}

int64_t lse_pack_bytes(int64_t P, int64_t T, int64_t H, int64_t Dv, int scatter_dim, cam_dtype dt)
{
    clear_error();
    PackGeom g;
    if (pack_geometry("lse_pack_bytes", P, T, H, Dv, scatter_dim, dt, &g) != CAM_OK)
        return -1;
    return g.total;
}

cam_status lse_pack(const void* out, int64_t o_sp, int64_t o_st, int64_t o_sh, const float* smax, int64_t m_sp,
                    int64_t m_st, int64_t m_sh, const float* ssum, int64_t s_sp, int64_t s_st, int64_t s_sh,
                    int64_t P, int64_t T, int64_t H, int64_t Dv, int scatter_dim, cam_dtype dt, void* packed,
                    void* stream)
{
    const char* op = "lse_pack";
    clear_error();
    PackGeom g;
    cam_status st = pack_geometry(op, P, T, H, Dv, scatter_dim, dt, &g);
    if (st != CAM_OK)
        return st;
    for (int64_t s : {o_sp, o_st, o_sh, m_sp, m_st, m_sh, s_sp, s_st, s_sh})
        if (s < 0 || s > kMaxStride)
            return set_error(CAM_ERR_UNSUPPORTED, "%s: strides must be non-negative and below 2^48", op);
    if (g.total == 0 || g.rows == 0)
        return CAM_OK;
    if (!out || !smax || !ssum || !packed)
        return set_error(CAM_ERR_NULL, "%s: out, softmax_max, softmax_sum and packed must be non-null", op);
    if (!aligned(out, 2) || !aligned(smax, 4) || !aligned(ssum, 4))
        return set_error(CAM_ERR_ALIGNMENT, "%s: out must be 2-byte and the statistics 4-byte aligned", op);
    if (!aligned(packed, 16))
        return set_error(CAM_ERR_ALIGNMENT, "%s: packed must be 16-byte aligned", op);
    int64_t e_o, e_m, e_s;
    if (!extent({P, T, H, Dv}, {o_sp, o_st, o_sh, 1}, 2, &e_o) || !extent({P, T, H}, {m_sp, m_st, m_sh}, 4, &e_m) ||
        !extent({P, T, H}, {s_sp, s_st, s_sh}, 4, &e_s))
        return set_error(CAM_ERR_SHAPE, "%s: tensor extent overflows", op);
    if (overlaps(packed, g.total, out, e_o) || overlaps(packed, g.total, smax, e_m) ||
        overlaps(packed, g.total, ssum, e_s))
        return set_error(CAM_ERR_OVERLAP, "%s: packed overlaps an input", op);
    if (P > 65535)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: P must be below 65536", op);

    Pack a{};
    const uint64_t row_b = uint64_t(Dv) * 2;
    a.width = pick_width({row_b == 0 ? 16 : row_b, reinterpret_cast<uintptr_t>(out), uint64_t(o_sp) * 2,
                          uint64_t(o_st) * 2, uint64_t(o_sh) * 2});
    a.out = out;
    a.o_sp_b = o_sp * 2;
    a.o_st_b = o_st * 2;
    a.o_sh_b = o_sh * 2;
    a.smax = smax;
    a.m_sp = m_sp;
    a.m_st = m_st;
    a.m_sh = m_sh;
    a.ssum = ssum;
    a.s_sp = s_sp;
    a.s_st = s_st;
    a.s_sh = s_sh;
    a.packed = packed;
    a.P = uint32_t(P);
    a.div_P = make_fastdiv(a.P);
    a.scatter_heads = scatter_dim == 1;
    a.inner = uint32_t(scatter_dim == 1 ? H / P : H);
    if (g.rows > INT32_MAX || a.inner == 0)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: rows per chunk must be below 2^31", op);
    a.div_inner = make_fastdiv(a.inner);
    a.Tp = uint64_t(T / P);
    a.Hp = uint32_t(H / P);
    a.rows = uint32_t(g.rows);
    if (row_b / a.width >= kU32Limit)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: one row exceeds 2^31 vectors", op);
    a.cv = uint32_t(row_b / a.width);
    a.div_cv = make_fastdiv(a.cv ? a.cv : 1);
    a.chunk_b = uint64_t(g.chunk);
    a.o_region_b = uint64_t(g.o_region);
    const uint64_t o_vecs = uint64_t(g.rows) * a.cv;
    if (o_vecs >= kU32Limit)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: one chunk exceeds 2^31 vectors", op);
    a.o_vecs = uint32_t(o_vecs);
    a.o_tiles_per_chunk = tiles(o_vecs, kPackTileVecs);
    a.div_otpc = make_fastdiv(a.o_tiles_per_chunk ? a.o_tiles_per_chunk : 1);
    a.l_tiles_per_chunk = tiles(uint64_t(g.rows), kThreads);
    a.div_ltpc = make_fastdiv(a.l_tiles_per_chunk);
    const uint64_t n_o = uint64_t(P) * uint64_t(P) * a.o_tiles_per_chunk;
    const uint64_t n_l = uint64_t(P) * uint64_t(P) * a.l_tiles_per_chunk;
    if (n_o + n_l > UINT32_MAX)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: more than 2^32 tiles", op);
    a.n_o_tiles = uint32_t(n_o);
    a.n_l_tiles = uint32_t(n_l);
    return launch_pack(a, stream);
}

cam_status lse_combine_packed(const void* packed, int64_t P, int64_t T, int64_t H, int64_t Dv, int scatter_dim,
                              cam_dtype dt, void* out, float* lse_out, void* stream)
{
    const char* op = "lse_combine_packed";
    clear_error();
    PackGeom g;
    cam_status st = pack_geometry(op, P, T, H, Dv, scatter_dim, dt, &g);
    if (st != CAM_OK)
        return st;
    if (g.total == 0 || g.rows == 0)
        return CAM_OK;
    if (!packed || !out)
        return set_error(CAM_ERR_NULL, "%s: packed and out must be non-null", op);
    if (!aligned(packed, 16))
        return set_error(CAM_ERR_ALIGNMENT, "%s: packed must be 16-byte aligned", op);
    // Destination rank r reads chunk (p, r) of every source p: as a strided
    // [P_src][P_dst][rows][Dv] view, p strides P chunks, r one chunk.
    CombineIn c{};
    c.po = packed;
    c.po_sp = P * g.chunk / 2;
    c.po_st = g.chunk / 2;
    c.po_sh = Dv;
    c.pl = reinterpret_cast<const float*>(static_cast<const char*>(packed) + g.o_region);
    c.pl_sp = P * g.chunk / 4;
    c.pl_st = g.chunk / 4;
    c.pl_sh = 1;
    c.P = P;
    c.T = P;
    c.H = g.rows;
    c.D = Dv;
    c.dt = dt;
    c.out = out;
    c.o_st = g.rows * Dv;
    c.o_sh = Dv;
    c.lse_out = lse_out;
    c.lo_st = g.rows;
    c.lo_sh = 1;
    return combine(op, c, stream);
}

cam_status lse_combine(const void* part_out, int64_t po_sp, int64_t po_st, int64_t po_sh, const float* part_lse,
                       int64_t pl_sp, int64_t pl_st, int64_t pl_sh, int64_t P, int64_t T, int64_t H, int64_t D,
                       cam_dtype dt, void* out, int64_t o_st, int64_t o_sh, float* lse_out, int64_t lo_st,
                       int64_t lo_sh, void* stream)
{
    clear_error();
    CombineIn c{part_out, po_sp, po_st, po_sh, part_lse, pl_sp, pl_st, pl_sh, P, T, H, D, dt,
                out, o_st, o_sh, lse_out, lo_st, lo_sh, nullptr, 0};
    return combine("lse_combine", c, stream);
}

cam_status lse_combine_varlen(const void* part_out, int64_t po_sp, int64_t po_st, int64_t po_sh,
                              const float* part_lse, int64_t pl_sp, int64_t pl_st, int64_t pl_sh, int64_t P,
                              int64_t T, int64_t H, int64_t D, cam_dtype dt, void* out, int64_t o_st, int64_t o_sh,
                              float* lse_out, int64_t lo_st, int64_t lo_sh, const int32_t* cu_seqlens,
                              int64_t nseq, void* stream)
{
    clear_error();
    if (T > 0 && !cu_seqlens)
        return set_error(CAM_ERR_NULL, "lse_combine_varlen: cu_seqlens must be non-null");
    CombineIn c{part_out, po_sp, po_st, po_sh, part_lse, pl_sp, pl_st, pl_sh, P, T, H, D, dt,
                out, o_st, o_sh, lse_out, lo_st, lo_sh, cu_seqlens, nseq};
    return combine("lse_combine_varlen", c, stream);
}

cam_status lse_combine_backward(const void* part_out, int64_t po_sp, int64_t po_st, int64_t po_sh,
                                const float* part_lse, int64_t pl_sp, int64_t pl_st, int64_t pl_sh, int64_t P,
                                int64_t T, int64_t H, int64_t D, cam_dtype dt, const void* g_out, int64_t go_st,
                                int64_t go_sh, const float* g_lse, int64_t gl_st, int64_t gl_sh, void* d_part_out,
                                int64_t dpo_sp, int64_t dpo_st, int64_t dpo_sh, float* d_part_lse, int64_t dpl_sp,
                                int64_t dpl_st, int64_t dpl_sh, void* stream)
{
    clear_error();
    CombineBwdIn c{part_out, po_sp, po_st, po_sh, part_lse, pl_sp, pl_st, pl_sh, P, T, H, D, dt,
                   g_out, go_st, go_sh, g_lse, gl_st, gl_sh, d_part_out, dpo_sp, dpo_st, dpo_sh,
                   d_part_lse, dpl_sp, dpl_st, dpl_sh, nullptr, 0};
    return combine_backward("lse_combine_backward", c, stream);
}

cam_status lse_combine_varlen_backward(const void* part_out, int64_t po_sp, int64_t po_st, int64_t po_sh,
                                       const float* part_lse, int64_t pl_sp, int64_t pl_st, int64_t pl_sh,
                                       int64_t P, int64_t T, int64_t H, int64_t D, cam_dtype dt, const void* g_out,
                                       int64_t go_st, int64_t go_sh, const float* g_lse, int64_t gl_st,
                                       int64_t gl_sh, void* d_part_out, int64_t dpo_sp, int64_t dpo_st,
                                       int64_t dpo_sh, float* d_part_lse, int64_t dpl_sp, int64_t dpl_st,
                                       int64_t dpl_sh, const int32_t* cu_seqlens, int64_t nseq, void* stream)
{
    clear_error();
    if (T > 0 && !cu_seqlens)
        return set_error(CAM_ERR_NULL, "lse_combine_varlen_backward: cu_seqlens must be non-null");
    if (T > INT32_MAX)
        return set_error(CAM_ERR_SHAPE, "lse_combine_varlen_backward: total_tokens must fit int32");
    CombineBwdIn c{part_out, po_sp, po_st, po_sh, part_lse, pl_sp, pl_st, pl_sh, P, T, H, D, dt,
                   g_out, go_st, go_sh, g_lse, gl_st, gl_sh, d_part_out, dpo_sp, dpo_st, dpo_sh,
                   d_part_lse, dpl_sp, dpl_st, dpl_sh, cu_seqlens, nseq};
    return combine_backward("lse_combine_varlen_backward", c, stream);
}

cam_status lse_combine_planned(const void* part_out, int64_t po_sp, int64_t po_st, int64_t po_sh,
                               const float* part_lse, int64_t pl_sp, int64_t pl_st, int64_t pl_sh, int64_t P,
                               int64_t T, int64_t H, int64_t D, cam_dtype dt, void* out, int64_t o_st, int64_t o_sh,
                               float* lse_out, int64_t lo_st, int64_t lo_sh, const int32_t* cu_seqlens,
                               const int32_t* first_pos, int64_t nseq, void* stream)
{
    clear_error();
    if (T > 0 && (!cu_seqlens || !first_pos))
        return set_error(CAM_ERR_NULL, "lse_combine_planned: cu_seqlens and first_pos must be non-null");
    if (T > INT32_MAX)
        return set_error(CAM_ERR_SHAPE, "lse_combine_planned: total_tokens must fit int32");
    CombineIn c{part_out, po_sp, po_st, po_sh, part_lse, pl_sp, pl_st, pl_sh, P, T, H, D, dt,
                out, o_st, o_sh, lse_out, lo_st, lo_sh, cu_seqlens, nseq};
    c.first = first_pos;
    return combine("lse_combine_planned", c, stream);
}

cam_status lse_combine_planned_backward(const void* part_out, int64_t po_sp, int64_t po_st, int64_t po_sh,
                                        const float* part_lse, int64_t pl_sp, int64_t pl_st, int64_t pl_sh,
                                        int64_t P, int64_t T, int64_t H, int64_t D, cam_dtype dt,
                                        const void* g_out, int64_t go_st, int64_t go_sh, const float* g_lse,
                                        int64_t gl_st, int64_t gl_sh, void* d_part_out, int64_t dpo_sp,
                                        int64_t dpo_st, int64_t dpo_sh, float* d_part_lse, int64_t dpl_sp,
                                        int64_t dpl_st, int64_t dpl_sh, const int32_t* cu_seqlens,
                                        const int32_t* first_pos, int64_t nseq, void* stream)
{
    clear_error();
    if (T > 0 && (!cu_seqlens || !first_pos))
        return set_error(CAM_ERR_NULL, "lse_combine_planned_backward: cu_seqlens and first_pos must be non-null");
    if (T > INT32_MAX)
        return set_error(CAM_ERR_SHAPE, "lse_combine_planned_backward: total_tokens must fit int32");
    CombineBwdIn c{part_out, po_sp, po_st, po_sh, part_lse, pl_sp, pl_st, pl_sh, P, T, H, D, dt,
                   g_out, go_st, go_sh, g_lse, gl_st, gl_sh, d_part_out, dpo_sp, dpo_st, dpo_sh,
                   d_part_lse, dpl_sp, dpl_st, dpl_sh, cu_seqlens, nseq};
    c.first = first_pos;
    return combine_backward("lse_combine_planned_backward", c, stream);
}

cam_status lse_combine_packed_seq(const void* packed, int64_t P, int64_t T, int64_t H, int64_t Dv, int scatter_dim,
                                  cam_dtype dt, void* out, float* lse_out, void* stream)
{
    const char* op = "lse_combine_packed_seq";
    clear_error();
    PackGeom g;
    cam_status st = pack_geometry(op, P, T, H, Dv, scatter_dim, dt, &g);
    if (st != CAM_OK)
        return st;
    if (g.total == 0 || g.rows == 0)
        return CAM_OK;
    if (!packed || !out)
        return set_error(CAM_ERR_NULL, "%s: packed and out must be non-null", op);
    if (!aligned(packed, 16))
        return set_error(CAM_ERR_ALIGNMENT, "%s: packed must be 16-byte aligned", op);
    if (P > INT32_MAX || H > INT32_MAX)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: P and H must fit 32 bits", op);
    // the exchange view as in lse_combine_packed; the output (extent T*H*Dv)
    // is placed token-major by out_mode 1 (head scatter) -- for the token
    // scatter the destination-major order already is token-major
    CombineIn c{};
    c.po = packed;
    c.po_sp = P * g.chunk / 2;
    c.po_st = g.chunk / 2;
    c.po_sh = Dv;
    c.pl = reinterpret_cast<const float*>(static_cast<const char*>(packed) + g.o_region);
    c.pl_sp = P * g.chunk / 4;
    c.pl_st = g.chunk / 4;
    c.pl_sh = 1;
    c.P = P;
    c.T = P;
    c.H = g.rows;
    c.D = Dv;
    c.dt = dt;
    c.out = out;
    c.o_st = g.rows * Dv;
    c.o_sh = Dv;
    c.lse_out = lse_out;
    c.lo_st = g.rows;
    c.lo_sh = 1;
    if (scatter_dim == 1) {
        c.out_mode = 1;
        c.Hp = H / P;
        c.Hq = H;
    }
    return combine(op, c, stream);
}

cam_status lse_combine_varlen_seq(const void* part_out, int64_t po_sp, int64_t po_st, int64_t po_sh,
                                  const float* part_lse, int64_t pl_sp, int64_t pl_st, int64_t pl_sh, int64_t P,
                                  int64_t T, int64_t H, int64_t D, cam_dtype dt, void* out, float* lse_out,
                                  const int32_t* cu_seqlens, const int32_t* rank_cu, const int64_t* rank_off,
                                  int64_t nseq, void* stream)
{
    const char* op = "lse_combine_varlen_seq";
    clear_error();
    if (T > 0 && (!cu_seqlens || !rank_cu || !rank_off))
        return set_error(CAM_ERR_NULL, "%s: cu_seqlens, rank_cu and rank_off must be non-null", op);
    if ((rank_cu && !aligned(rank_cu, 4)) || (rank_off && !aligned(rank_off, 8)))
        return set_error(CAM_ERR_ALIGNMENT, "%s: misaligned plan array", op);
    int64_t hd = 0;
    if (P > 0 && nseq >= 0 && T > 0 && D >= 0 && H >= 0) {
        int64_t ob, lb = 0, rcb, rob;
        if (!prod_ok({T, H, D, 2}, &ob) || (lse_out && !prod_ok({T, H, 4}, &lb)) || nseq == kI64Max ||
            !prod_ok({P, nseq + 1, 4}, &rcb) || P == kI64Max || !prod_ok({P + 1, 8}, &rob) || !prod_ok({H, D}, &hd))
            return set_error(CAM_ERR_SHAPE, "%s: sizes overflow", op);
        if (overlaps(out, ob, rank_cu, rcb) || overlaps(out, ob, rank_off, rob) || overlaps(lse_out, lb, rank_cu, rcb) ||
            overlaps(lse_out, lb, rank_off, rob))
            return set_error(CAM_ERR_OVERLAP, "%s: an output overlaps the plan arrays", op);
    }
    CombineIn c{part_out, po_sp, po_st, po_sh, part_lse, pl_sp, pl_st, pl_sh, P, T, H, D, dt,
                out, hd, D, lse_out, H, 1, cu_seqlens, nseq};
    c.out_mode = 2;
    c.rank_cu = rank_cu;
    c.rank_off = rank_off;
    return combine(op, c, stream);
}

cam_status lse_merge(float* acc_out, int64_t a_st, int64_t a_sh, float* acc_lse, int64_t al_st, int64_t al_sh,
                     const void* part_out, int64_t p_st, int64_t p_sh, const float* part_lse, int64_t pl_st,
                     int64_t pl_sh, int64_t T, int64_t H, int64_t D, cam_dtype dt, void* out_final, int64_t f_st,
                     int64_t f_sh, void* stream)
{
    const char* op = "lse_merge";
    clear_error();
    if (T < 0 || H < 0 || D < 0)
        return set_error(CAM_ERR_SHAPE, "%s: need T, H, D >= 0", op);
    if (dt != CAM_BF16 && dt != CAM_FP16)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: payload dtype must be bf16 or fp16", op);
    for (int64_t s : {a_st, a_sh, al_st, al_sh, p_st, p_sh, pl_st, pl_sh, f_st, f_sh})
        if (s < 0 || s > kMaxStride)
            return set_error(CAM_ERR_UNSUPPORTED, "%s: strides must be non-negative and below 2^48", op);
    int64_t n_rows;
    if (!prod_ok({T, H}, &n_rows))
        return set_error(CAM_ERR_SHAPE, "%s: T*H overflows", op);
    if (n_rows == 0)
        return CAM_OK;
    if (n_rows > INT32_MAX)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: T*H must be below 2^31 rows", op);
    if (!acc_out || !acc_lse || !part_out || !part_lse)
        return set_error(CAM_ERR_NULL, "%s: accumulator and partial pointers must be non-null", op);
    if (D % 4)
        return set_error(CAM_ERR_ALIGNMENT, "%s: D must be a multiple of 4 (4-element accesses)", op);
    if (!aligned(acc_out, 16) || a_st % 4 || a_sh % 4 || !aligned(part_out, 8) || p_st % 4 || p_sh % 4 ||
        !aligned(acc_lse, 4) || !aligned(part_lse, 4) ||
        (out_final && (!aligned(out_final, 8) || f_st % 4 || f_sh % 4)))
        return set_error(CAM_ERR_ALIGNMENT, "%s: rows must start 16-byte (accumulator) / 8-byte (payload) aligned", op);
    int64_t e_a, e_al, e_p, e_pl, e_f = 0;
    if (!extent({T, H, D}, {a_st, a_sh, 1}, 4, &e_a) || !extent({T, H}, {al_st, al_sh}, 4, &e_al) ||
        !extent({T, H, D}, {p_st, p_sh, 1}, 2, &e_p) || !extent({T, H}, {pl_st, pl_sh}, 4, &e_pl) ||
        (out_final && !extent({T, H, D}, {f_st, f_sh, 1}, 2, &e_f)))
        return set_error(CAM_ERR_SHAPE, "%s: tensor extent overflows", op);
    if (overlaps(acc_out, e_a, part_out, e_p) || overlaps(acc_out, e_a, part_lse, e_pl) ||
        overlaps(acc_lse, e_al, part_out, e_p) || overlaps(acc_lse, e_al, part_lse, e_pl) ||
        overlaps(acc_out, e_a, acc_lse, e_al) || overlaps(out_final, e_f, acc_out, e_a) ||
        overlaps(out_final, e_f, acc_lse, e_al) || overlaps(out_final, e_f, part_out, e_p) ||
        overlaps(out_final, e_f, part_lse, e_pl))
        return set_error(CAM_ERR_OVERLAP, "%s: buffers overlap", op);
    Merge a{};
    a.acc = acc_out;
    a.a_st = a_st;
    a.a_sh = a_sh;
    a.acc_lse = acc_lse;
    a.al_st = al_st;
    a.al_sh = al_sh;
    a.part = part_out;
    a.p_st_b = p_st * 2;
    a.p_sh_b = p_sh * 2;
    a.part_lse = part_lse;
    a.pl_st = pl_st;
    a.pl_sh = pl_sh;
    a.fin = out_final;
    a.f_st_b = f_st * 2;
    a.f_sh_b = f_sh * 2;
    a.H = uint32_t(H);
    a.div_H = make_fastdiv(a.H);
    a.n_rows = uint64_t(n_rows);
    if (uint64_t(D / 4) >= kU32Limit)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: one row exceeds 2^31 vectors", op);
    a.cv = uint32_t(D / 4);
    a.g_log2 = log2u(pow2ceil(a.cv < 64 ? (a.cv ? a.cv : 1) : 64));
    if (a.g_log2 < 6 && kCombineNarrowVpl == 2 && a.g_log2 > 0)
        a.g_log2 -= 1;  // narrow rows: each lane moves two vectors of the row per pass
    a.fp16 = dt == CAM_FP16;
    return launch_merge(a, stream);
}

cam_status qkv_projection_head_sharded(const void* x, const void* w, void* out, int64_t S, int64_t K, int64_t P,
                                       int64_t B, int64_t H, int64_t D, cam_dtype dt, void* stream)
{
    const char* op = "qkv_projection_head_sharded";
    clear_error();
    if (S < 0 || K < 0 || P < 1 || B < 0 || H < 0 || D < 0)
        return set_error(CAM_ERR_SHAPE, "%s: need P >= 1 and S, K, B, H, D >= 0", op);
    if (dt != CAM_BF16 && dt != CAM_FP16)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: operands must be bf16 or fp16", op);
    if (H % P)
        return set_error(CAM_ERR_DIVISIBILITY, "%s: H (%lld) must be a multiple of P (%lld)", op, (long long)H,
                         (long long)P);
    int64_t N, xb, wb, ob;
    if (!prod_ok({B, H, D}, &N) || !prod_ok({S, K, 2}, &xb) || !prod_ok({N, K, 2}, &wb) || !prod_ok({S, N, 2}, &ob))
        return set_error(CAM_ERR_SHAPE, "%s: sizes overflow", op);
    if (S == 0 || N == 0)
        return CAM_OK;
    if (K == 0 || K % 64 || N % 256)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: needs K a positive multiple of 64 and B*H*D a multiple of 256", op);
    if (S > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
        return set_error(CAM_ERR_UNSUPPORTED, "%s: S, K and B*H*D must be below 2^31", op);
    if (!x || !w || !out)
        return set_error(CAM_ERR_NULL, "%s: x, w and out must be non-null", op);
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(out, 2))
        return set_error(CAM_ERR_ALIGNMENT, "%s: x and w must be 16-byte aligned, out 2-byte aligned", op);
    if (overlaps(out, ob, x, xb) || overlaps(out, ob, w, wb))
        return set_error(CAM_ERR_OVERLAP, "%s: out overlaps an operand", op);
    Proj a{};
    a.x = x;
    a.w = w;
    a.out = out;
    a.M = uint32_t(S);
    a.K = uint32_t(K);
    a.S = uint32_t(S);
    a.B = uint32_t(B);
    a.HD = uint32_t(H * D);
    a.HpD = uint32_t((H / P) * D);
    if (a.HpD == 0)
        return CAM_OK;
    a.div_HD = make_fastdiv(a.HD);
    a.div_HpD = make_fastdiv(a.HpD);
    a.tiles_m = uint32_t((S + 255) / 256);
    a.tiles_n = uint32_t(N / 256);
    if (uint64_t(a.tiles_m) * a.tiles_n > (1u << 20))
        return set_error(CAM_ERR_UNSUPPORTED, "%s: more than 2^20 output tiles", op);
    a.group_m = CAM_PROJ_GROUP_M;
    a.vec_out = (CAM_PROJ_VEC_OUT && a.HpD % 8 == 0 && aligned(out, 16)) ? 1 : 0;
    a.fp16 = dt == CAM_FP16;
    return launch_proj(a, stream);
}

cam_status cam_copy(const void* src, void* dst, int64_t bytes, void* stream)
{
    clear_error();
    if (bytes < 0)
        return set_error(CAM_ERR_SHAPE, "cam_copy: bytes must be >= 0");
    if (bytes == 0)
        return CAM_OK;
    if (!src || !dst)
        return set_error(CAM_ERR_NULL, "cam_copy: src and dst must be non-null");
    if (!aligned(src, 16) || !aligned(dst, 16) || bytes % 16)
        return set_error(CAM_ERR_ALIGNMENT, "cam_copy: 16-byte aligned pointers and size required");
    if (overlaps(src, bytes, dst, bytes))
        return set_error(CAM_ERR_OVERLAP, "cam_copy: src and dst overlap");
    Copy a{src, dst, uint64_t(bytes) / 16};
    return launch_copy(a, stream);
}

}  // extern "C"
