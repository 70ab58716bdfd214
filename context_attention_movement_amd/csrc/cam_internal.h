// cam_internal.h -- shared internals of libcam: the launch records the host
// layer fills after validation, and division by run-time invariant integers.
//
// This header is included by the host-only API layer (cam_api.cpp, compiled
// without any HIP call) and by the kernel sources (*.hip).
#pragma once

#include <stdint.h>

#include "cam.h"

namespace cam {

// Unsigned 32-bit division by a run-time invariant d >= 1 with one high
// multiply, one add and one shift (Granlund & Montgomery, "Division by
// invariant integers using multiplication", PLDI 1994, section 4):
//   l = ceil(log2 d),  m = floor(2^32 (2^l - d) / d) + 1,
//   n / d = (umulhi(n, m) + n) >> l   for every 0 <= n < 2^32,
// the add taken in 64 bits so that it cannot wrap.
struct FastDiv {
    uint32_t d;
    uint32_t m;
    uint32_t l;
};

inline FastDiv make_fastdiv(uint32_t d)
{
    FastDiv f;
    f.d = d;
    uint32_t l = 0;
    while (l < 32 && (uint64_t(1) << l) < d)
        ++l;
    f.l = l;
    f.m = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
    return f;
}

// ---------------------------------------------------------------------------
// Launch records: everything a kernel needs, computed and checked on the host.
// Offsets and strides named *_b are in bytes; vector counts in units of the
// access width W chosen for the launch.
// ---------------------------------------------------------------------------

// Dense relayout.  A slab is (r, b, j): the S/P rows moving between rank j's
// sequence shard and rank r's head shard of plane b.  Slab index
// ((r*B + b)*P + j) orders the head side exactly as it lies in memory, so the
// head side of slab k starts at vector k*slab_vecs; its sequence side starts at
// ((j*B + b)*(S/P)*P + r)*c with consecutive rows P*c vectors apart.
struct DenseRelayout {
    const void* src;
    void* dst;
    uint32_t P, B;
    FastDiv div_P, div_B;
    uint32_t c;            // vectors per row run ((H/P)*D*esize / W)
    FastDiv div_c;
    uint64_t Pc;           // sequence-side row stride in vectors (P*c)
    uint64_t Sp;           // rows per slab (S/P)
    uint32_t slab_vecs;    // Sp*c
    uint32_t tiles_per_slab;
    FastDiv div_tps;
    uint32_t n_tiles;      // P*B*P*tiles_per_slab
    int width;             // W in bytes: 16, 8, 4 or 2
    bool seq_to_head;
};

// Varlen relayout.  A plane is (r, b); the head side of plane (r, b) is rows
// t < T of c vectors each, contiguous at vector (r*B + b)*T*c.  Token t's
// sequence-side row is found per tile from cu_seqlens and the plan.
// With spans set, cu holds the planned spans' first tokens (nseq = number of
// spans, cu[nseq] = T) and token t of span s is row span_local[s] + t - cu[s]
// of rank span_rank[s]'s slab (a THD layout plan) instead of a piece of the
// per-sequence split.
struct VarlenRelayout {
    const void* src;
    void* dst;
    const int32_t* cu;
    const int32_t* rank_cu;
    const int64_t* rank_off;
    const int32_t* span_rank;
    const int32_t* span_local;
    bool spans;
    int32_t nseq;
    uint32_t P, B;
    FastDiv div_P, div_B;
    uint64_t T;
    uint32_t c;
    FastDiv div_c;
    uint64_t Pc;
    uint64_t plane_vecs;    // T*c
    uint32_t tiles_per_plane;
    FastDiv div_tpp;
    uint32_t n_tiles;
    int width;
    bool seq_to_head;
};

// Max/sum-aware LSE pack.
struct Pack {
    const void* out;
    int64_t o_sp_b, o_st_b, o_sh_b;
    const float* smax;
    int64_t m_sp, m_st, m_sh;
    const float* ssum;
    int64_t s_sp, s_st, s_sh;
    void* packed;
    uint32_t P;
    FastDiv div_P;
    uint32_t scatter_heads; // 1: scatter_dim 1 (heads), 0: scatter_dim 0 (tokens)
    uint32_t inner;         // H/P (heads) or H (tokens): row q = outer*inner + inner_idx
    FastDiv div_inner;
    uint64_t Tp;            // T/P (tokens) -- token offset of destination r is r*Tp
    uint32_t Hp;            // H/P (heads)
    uint32_t rows;          // rows per chunk
    uint32_t cv;            // vectors per row (Dv*esize / W)
    FastDiv div_cv;
    uint64_t chunk_b, o_region_b;
    uint32_t o_vecs;        // rows*cv per chunk
    uint32_t o_tiles_per_chunk;
    FastDiv div_otpc;
    uint32_t n_o_tiles;     // P*P*o_tiles_per_chunk
    uint32_t l_tiles_per_chunk;
    FastDiv div_ltpc;
    uint32_t n_l_tiles;     // P*P*l_tiles_per_chunk
    int width;
};

// Stable LSE combine over rows (t, h).
struct Combine {
    const void* po;
    int64_t po_sp_b, po_st_b, po_sh_b;
    const float* pl;
    int64_t pl_sp, pl_st, pl_sh;
    void* out;
    int64_t o_st_b, o_sh_b;
    float* lse_out;
    int64_t lo_st, lo_sh;
    uint32_t P;
    uint32_t H;
    FastDiv div_H;
    uint64_t n_rows;        // T*H
    uint32_t cv;            // vectors per row
    uint32_t g_log2;        // payload lanes per row = 1 << g_log2 (<= 64)
    uint32_t gp_log2;       // statistics lanes per row = 1 << gp_log2 (>= P, <= 64)
    uint32_t rows_per_tile; // rows per workgroup tile
    uint64_t n_tiles;
    uint32_t threads;       // workgroup size (64, 128 or 256)
    uint32_t xcd;           // 1: XCD-aware tile order
    // output placement of row (t, h):
    //   0: out + t*o_st_b + h*o_sh_b, lse_out + t*lo_st + h*lo_sh
    //   1: the exchange view's row (r = t, q = h) goes to token-major row
    //      g = (q / Hp)*Hq + r*Hp + q % Hp  (head scatter: [T][H][Dv])
    //   2: token t goes to its rank-major (sequence-sharded) row of a packed
    //      THD batch, from cu_seqlens and the varlen plan: g = row*H + h
    uint32_t out_mode;
    uint32_t Hp, Hq;        // mode 1: heads per rank, heads in total
    FastDiv div_Hp;
    uint64_t o_row_b;       // modes 1, 2: bytes per output row
    const int32_t* rank_cu; // mode 2: the varlen plan
    const int64_t* rank_off;
    const int32_t* cu;      // non-null: causal gating (varlen)
    const int32_t* first;   // with cu: a plan's first positions [P][nseq]; null: piece rule
    int32_t nseq;
    FastDiv div_P;
    int width;
    int fp16;               // payload: 0 bf16, 1 fp16
};

// Online two-way merge: accumulator (fp32 payload + fp32 LSE) <- stable
// combine of itself and one partial.  Rows (t, h); a lane moves 4 elements.
struct Merge {
    float* acc;
    int64_t a_st, a_sh;     // element strides (4-element aligned)
    float* acc_lse;
    int64_t al_st, al_sh;
    const void* part;
    int64_t p_st_b, p_sh_b; // byte strides
    const float* part_lse;
    int64_t pl_st, pl_sh;
    void* fin;              // optional rounded payload (nullable)
    int64_t f_st_b, f_sh_b;
    uint32_t H;
    FastDiv div_H;
    uint64_t n_rows;
    uint32_t cv;            // 4-element chunks per row
    uint32_t g_log2;        // lanes per row
    int fp16;
};

// Gradient of the combine: for each row (t, h), from the partials, their
// LSEs and the upstream gradients (g of the output row, g_lse of its LSE),
// dO_p = w_p g and dL_p = w_p (<g, O_p> - <g, out> + g_lse) over the valid
// partials, zero for the others.
struct CombineBwd {
    const void* po;
    int64_t po_sp_b, po_st_b, po_sh_b;
    const float* pl;
    int64_t pl_sp, pl_st, pl_sh;
    const void* go;         // upstream gradient of out (payload dtype)
    int64_t go_st_b, go_sh_b;
    const float* gl;        // upstream gradient of lse_out (nullable: zero)
    int64_t gl_st, gl_sh;
    void* dpo;              // gradient of the partial outputs (payload dtype)
    int64_t dpo_sp_b, dpo_st_b, dpo_sh_b;
    float* dpl;             // gradient of the partial LSEs
    int64_t dpl_sp, dpl_st, dpl_sh;
    uint32_t P;
    uint32_t H;
    FastDiv div_H;
    uint64_t n_rows;
    uint32_t cv;
    uint32_t g_log2;
    uint32_t gp_log2;
    uint32_t rows_per_tile;
    uint64_t n_tiles;
    const int32_t* cu;      // non-null: causal gating (varlen)
    const int32_t* first;   // with cu: a plan's first positions [P][nseq]; null: piece rule
    int32_t nseq;
    FastDiv div_P;
    int width;
    int fp16;
    uint32_t threads;       // workgroup size
    uint32_t compact;       // 1: compacted partial lists and LDS-reduced dot products (see lse.hip)
};

// Q/K/V projection into the head-sharded layout: out[r][b][t][h'][d] =
// sum_k x[t][k] w[(b*H + r*Hp + h')*D + d][k] (MFMA, 256 x 256 tiles).
struct Proj {
    const void* x;          // [M = S][K]
    const void* w;          // [N = B*H*D][K]
    void* out;              // [P][B][S][Hp][D]
    uint32_t M, K;
    uint32_t S, B;
    uint32_t HD, HpD;       // H*D, (H/P)*D
    FastDiv div_HD, div_HpD;
    uint32_t tiles_m, tiles_n, group_m;
    int vec_out;            // 1: 16-byte output segments through LDS ((H/P)*D % 8 == 0, out 16-byte aligned)
    int fp16;
};

struct Copy {
    const void* src;
    void* dst;
    uint64_t n_vecs;        // 16-byte vectors
};

// LDS-staged seq->head relayout (an ablation measured against the direct
// kernel; ulysses_seq_to_head does not use it).  A tile is R consecutive
// sequence-side rows (all H heads, R*P*c contiguous vectors) of one (j, b)
// slab, staged whole in LDS and written as P contiguous runs of R*c vectors.
struct DenseLds {
    const void* src;
    void* dst;
    uint32_t P, B;
    uint32_t c;             // vectors per head-block run
    FastDiv div_c;
    uint32_t R;             // rows per tile
    uint32_t Rc;            // R*c
    FastDiv div_Rc;
    uint64_t Sp;            // rows per source slab (S/P)
    uint32_t tiles_per_slab;  // ceil(Sp / R)
    FastDiv div_tps;
    FastDiv div_B;
    uint32_t n_tiles;       // P*B*tiles_per_slab
};

// Kernel launchers (defined in the .hip sources).  They only launch; the
// records have been validated.  Return CAM_OK or CAM_ERR_HIP (message set).
cam_status launch_dense_relayout(const DenseRelayout& a, void* stream);
cam_status launch_varlen_relayout(const VarlenRelayout& a, void* stream);
cam_status launch_pack(const Pack& a, void* stream);
cam_status launch_combine(const Combine& a, void* stream);
cam_status launch_copy(const Copy& a, void* stream);
cam_status launch_dense_lds(const DenseLds& a, void* stream);
cam_status launch_merge(const Merge& a, void* stream);
cam_status launch_combine_bwd(const CombineBwd& a, void* stream);
cam_status launch_proj(const Proj& a, void* stream);

// Error reporting shared by the host layer and the launchers.
cam_status set_error(cam_status s, const char* fmt, ...);
// records the geometry of this thread's latest launch (cam_last_launch)
void note_launch(uint64_t workgroups, uint32_t threads, uint64_t lds_bytes);
void clear_error();

// cu_seqlens entries staged in LDS by the varlen kernels (larger tables are
// searched in global memory, 64 entries per step by a whole wave).
constexpr int32_t kCuCache = 1024;

// Launch shape shared by all streaming kernels.
#ifndef CAM_THREADS
#define CAM_THREADS 256
#endif
constexpr int kThreads = CAM_THREADS;
// 16-byte vectors each thread moves per tile (its loads all in flight before
// its stores): the pack's payload, the plain copy, the dense relayout, the
// varlen relayout -- chosen per kernel by measurement on MI355X with inputs
// too large for the Infinity Cache.
#ifndef CAM_VECS_PACK
#define CAM_VECS_PACK 3
#endif
constexpr int kPackVecs = CAM_VECS_PACK;
constexpr int kPackTileVecs = kThreads * kPackVecs;
#ifndef CAM_VECS_COPY
#define CAM_VECS_COPY 1
#endif
constexpr int kCopyVecs = CAM_VECS_COPY;
constexpr int kCopyTileVecs = kThreads * kCopyVecs;
#ifndef CAM_VECS_DENSE
#define CAM_VECS_DENSE 1
#endif
constexpr int kDenseVecs = CAM_VECS_DENSE;
constexpr int kDenseTileVecs = kThreads * kDenseVecs;
#ifndef CAM_VECS_VARLEN
#define CAM_VECS_VARLEN 4
#endif
constexpr int kVarlenVecs = CAM_VECS_VARLEN;
constexpr int kVarlenTileVecs = kThreads * kVarlenVecs;
// Non-temporal policy per kernel (bit 0: loads, bit 1: stores), chosen by
// measurement on MI355X.
#ifndef CAM_NT_SEQ_TO_HEAD
#define CAM_NT_SEQ_TO_HEAD 3
#endif
#ifndef CAM_NT_HEAD_TO_SEQ
#define CAM_NT_HEAD_TO_SEQ 3
#endif
#ifndef CAM_NT_VARLEN_SEQ_TO_HEAD
#define CAM_NT_VARLEN_SEQ_TO_HEAD 3
#endif
#ifndef CAM_NT_VARLEN_HEAD_TO_SEQ
#define CAM_NT_VARLEN_HEAD_TO_SEQ 3
#endif
#ifndef CAM_NT_PACK
#define CAM_NT_PACK 3
#endif
#ifndef CAM_NT_COMBINE
#define CAM_NT_COMBINE 3
#endif
#ifndef CAM_NT_COPY
#define CAM_NT_COPY 3
#endif
// gradient rows of >= 64 vectors by the LDS-free row-stream kernel (1) or the
// tiled kernel with shuffle-reduced dot products (0); the stream kernel's tile
// order (1 XCD-aware) and non-temporal policy (bit 0 loads, bit 1 stores)
#ifndef CAM_COMBINE_BWD_STREAM
#define CAM_COMBINE_BWD_STREAM 1
#endif
#ifndef CAM_XCD_COMBINE_BWD_STREAM
#define CAM_XCD_COMBINE_BWD_STREAM 1
#endif
#ifndef CAM_NT_COMBINE_BWD_STREAM
#define CAM_NT_COMBINE_BWD_STREAM 3
#endif
#ifndef CAM_NT_COMBINE_BWD
#define CAM_NT_COMBINE_BWD 2
#endif
#ifndef CAM_NT_MERGE
#define CAM_NT_MERGE 3
#endif
// Projection: row tiles per group of the tile order (column tiles of a
// group run close together in time and share their weight tiles in cache).
#ifndef CAM_PROJ_GROUP_M
#define CAM_PROJ_GROUP_M 32
#endif
// Projection epilogue: 16-byte output segments staged through LDS (1) or
// one 2-byte store per accumulator element (0)
// Projection LDS swizzle: chunk position XOR ((row >> shift) % 8)
#ifndef CAM_PROJ_SWZ_SHIFT
#define CAM_PROJ_SWZ_SHIFT 1
#endif
#ifndef CAM_PROJ_VEC_OUT
#define CAM_PROJ_VEC_OUT 1
#endif
// Combine gradient tiling: rows per tile for rows of >= 512 bytes and shorter.
// rounds of the tiled combines' first phase (one lane per (row, partial)) a
// tile may take: workgroups widen, then tiles shorten, for many partials
#ifndef CAM_COMBINE_STATS_ROUNDS
#define CAM_COMBINE_STATS_ROUNDS 4
#endif
#ifndef CAM_COMBINE_BWD_ROWS_WIDE
#define CAM_COMBINE_BWD_ROWS_WIDE 8
#endif
#ifndef CAM_COMBINE_BWD_ROWS_NARROW
#define CAM_COMBINE_BWD_ROWS_NARROW 16
#endif
#ifndef CAM_COMBINE_BWD_BATCH
#define CAM_COMBINE_BWD_BATCH 4
#endif
constexpr int kCombineBwdBatch = CAM_COMBINE_BWD_BATCH;
// gradient, compacted form: valid partial rows loaded at once per lane (1..8)
// and vectors of a row per lane per pass (1 or 2)
#ifndef CAM_COMBINE_BWD_NARROW_BATCH
#define CAM_COMBINE_BWD_NARROW_BATCH 1
#endif
#ifndef CAM_COMBINE_BWD_VPL
#define CAM_COMBINE_BWD_VPL 1
#endif
constexpr int kCombineBwdNarrowBatch = CAM_COMBINE_BWD_NARROW_BATCH;
constexpr int kCombineBwdVpl = CAM_COMBINE_BWD_VPL;
static_assert(kCombineBwdNarrowBatch >= 1 && kCombineBwdNarrowBatch <= 8, "gradient batch must be 1..8");
static_assert(kCombineBwdVpl == 1 || kCombineBwdVpl == 2, "gradient vectors per lane must be 1 or 2");
// Combine tiling (measured on MI355X): rows per workgroup tile for rows of
// >= 512 bytes and for shorter rows, and partial rows loaded per batch.
#ifndef CAM_COMBINE_ROWS_WIDE
#define CAM_COMBINE_ROWS_WIDE 8
#endif
#ifndef CAM_COMBINE_ROWS_NARROW
#define CAM_COMBINE_ROWS_NARROW 32
#endif
#ifndef CAM_COMBINE_BATCH
#define CAM_COMBINE_BATCH 4
#endif
constexpr int kCombineBatch = CAM_COMBINE_BATCH;
// rows of < 64 vectors: most valid partial rows loaded at once per lane
#ifndef CAM_COMBINE_NARROW_BATCH
#define CAM_COMBINE_NARROW_BATCH 1
#endif
constexpr int kCombineNarrowBatch = CAM_COMBINE_NARROW_BATCH;
static_assert(kCombineNarrowBatch >= 1 && kCombineNarrowBatch <= 8, "narrow combine batch must be 1..8");
// rows of < 64 vectors: vectors of a row each lane moves per pass (1 or 2);
// a row then takes pow2ceil(ceil(vectors / VPL)) lanes
#ifndef CAM_COMBINE_NARROW_VPL
#define CAM_COMBINE_NARROW_VPL 2
#endif
constexpr int kCombineNarrowVpl = CAM_COMBINE_NARROW_VPL;
static_assert(kCombineNarrowVpl == 1 || kCombineNarrowVpl == 2, "vectors per lane must be 1 or 2");
// rows of < 64 vectors: 1 = the valid partials one at a time, the next one's
// payload requested before the current one is accumulated (software pipeline)
#ifndef CAM_COMBINE_NARROW_PIPE
#define CAM_COMBINE_NARROW_PIPE 0
#endif
// rows of >= 64 vectors (a whole wave per row): rows per tile, rows in flight
// per wave, partial rows per batch
#ifndef CAM_COMBINE_THREADS_WAVE
#define CAM_COMBINE_THREADS_WAVE 64
#endif
#ifndef CAM_COMBINE_ROWS_WAVE
#define CAM_COMBINE_ROWS_WAVE 1
#endif
#ifndef CAM_COMBINE_INFLIGHT_WAVE
#define CAM_COMBINE_INFLIGHT_WAVE 1
#endif
#ifndef CAM_COMBINE_BATCH_WAVE
#define CAM_COMBINE_BATCH_WAVE 8
#endif
// rows of >= 64 vectors by the LDS-free row-stream kernel (1) or the tiled
// kernel (0); its workgroup size and rows per wave
#ifndef CAM_COMBINE_STREAM
#define CAM_COMBINE_STREAM 1
#endif
#ifndef CAM_COMBINE_STREAM_THREADS
#define CAM_COMBINE_STREAM_THREADS 64
#endif
#ifndef CAM_COMBINE_STREAM_ROWS
#define CAM_COMBINE_STREAM_ROWS 1
#endif
constexpr int kCombineInFlightWave = CAM_COMBINE_INFLIGHT_WAVE;
constexpr int kCombineBatchWave = CAM_COMBINE_BATCH_WAVE;
// XCD-aware tile order per kernel (1 = each XCD takes a contiguous range of
// tiles, 0 = hardware order), chosen by measurement on MI355X.
#ifndef CAM_XCD_SEQ_TO_HEAD
#define CAM_XCD_SEQ_TO_HEAD 1
#endif
#ifndef CAM_XCD_HEAD_TO_SEQ
#define CAM_XCD_HEAD_TO_SEQ 1
#endif
#ifndef CAM_XCD_VARLEN_SEQ_TO_HEAD
#define CAM_XCD_VARLEN_SEQ_TO_HEAD 0
#endif
#ifndef CAM_XCD_VARLEN_HEAD_TO_SEQ
#define CAM_XCD_VARLEN_HEAD_TO_SEQ 1
#endif
#ifndef CAM_XCD_MERGE
#define CAM_XCD_MERGE 0
#endif
#ifndef CAM_XCD_PACK
#define CAM_XCD_PACK 0
#endif
#ifndef CAM_XCD_COMBINE_WAVE
#define CAM_XCD_COMBINE_WAVE 1
#endif
#ifndef CAM_XCD_COMBINE_NARROW
#define CAM_XCD_COMBINE_NARROW 0
#endif
#ifndef CAM_XCD_COPY
#define CAM_XCD_COPY 1
#endif
#ifndef CAM_MAX_GRID
#define CAM_MAX_GRID (1u << 20)
#endif
constexpr uint32_t kMaxGrid = CAM_MAX_GRID;

}  // namespace cam
